"""Benchmarks of the streaming KV-cache attention path on one MI355X.

Default (one JSON line, the headline metric): the single streaming step --
P = 1374 tokens per frame (37x37 patches + 1 camera + 4 register), H = 16,
D = 64, bf16, 8 scale frames + a 16-frame window, so each step attends 1374
queries to 24 x 1374 = 32,976 keys.  One step = append (K and V into the
frame's ring page) + evict + attention (split pieces merged), through the
C ABI, returning the attention output (the pages' compute_attention returns
the output only; the time with an LSE output as well is reported beside).

  value        TFLOP/s of the whole step: algorithmic attention FLOPs
               (4*D*H*visible query-key pairs) / measured step time
  roofline     the dominant kernel against its bound: the attention call
               (timed with HIP events on the stream it runs on) against the
               bf16 dense MFMA peak; traffic is the HBM bytes per launch from
               the FETCH_SIZE/WRITE_SIZE counter summary under profiles/, or
               null when the kernel sources have changed since those counters
               were taken
  cpu_baseline the float64 oracle on the host cores, a bounded sample

--workload tiny | prefill | rope | specials | normed | decode | graph | all
prints the other workloads, each line with its own roofline and CPU baseline:
  tiny      6 frames of 21 tokens, H = 2, D = 32, fp32: masked prefill and a
            6-step stream (latency-bound; the fp32 vector-ALU kernel)
  prefill   32 frames at once (43,968 tokens), window 8, 8 scale frames
  rope      2000 frames streamed with 3-D RoPE, window 6 blocks x 4 frames,
            8 scale frames (steady state t >= 31)
  specials  1600 frames, P = 1405 (28x50 + 5), window 16, 8 scale frames,
            5 special rows of up to 1000 evicted frames retained, every
            third frame a non-keyframe (append, attend, roll back)
  normed    the rope stream's configuration with a per-head q/k layer
            norm fused into the RoPE + append pass, against the same steps
            run as a separate norm kernel followed by the RoPE + append
  decode    token decode, 32 query heads over 8 kv heads, a 4096-slot
            rolling buffer per sequence, batch 16 (and batch 1), buffer full
  graph     the headline step for 12 layers as one captured graph replayed
            per frame, against the same 12 layers stepped one call each

Kernel times of the HBM-bound passes (append, RoPE) are device times: the
stream is first held by a spin kernel so that the timed launches queue up
and run back to back, and each launch is bracketed by its own event pair.
A plain device-to-device copy of the same byte count, timed the same way,
gives the measured copy ceiling those passes are compared with.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16, published
FP32_VECTOR_PEAK_TFLOPS = 157.3     # MI355X fp32 vector, published
HBM_PEAK_GBS = 8000.0
METRIC = "attention TFLOP/s and frames/s per layer, streaming step (1374 q x ~33k keys)"


def _timed(torch, fn, steps):
    """Average ms per call of fn(i) over `steps` calls (events on the current stream)."""
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _per_step(torch, fn, idx):
    """Per-call ms of fn(i) for i in idx (one event pair per call)."""
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(idx) + 1)]
    ev[0].record()
    for j, i in enumerate(idx):
        fn(i)
        ev[j + 1].record()
    torch.cuda.synchronize()
    return [ev[j].elapsed_time(ev[j + 1]) for j in range(len(idx))]


def _device_ms(torch, fn, n=40, hold_cycles=4_000_000):
    """Median device time in ms of one launch of fn(i): the stream is held by
    a spin kernel while n (event, launch, event) triples are enqueued, so the
    launches run back to back and each event pair brackets one launch."""
    torch.cuda.synchronize()
    torch.cuda._sleep(hold_cycles)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2]


def _copy_ceiling_gbs(torch, moved_bytes):
    """GB/s of a plain device-to-device copy moving `moved_bytes` (half read, half written)."""
    n = moved_bytes // 2
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    ms = _device_ms(torch, lambda _: dst.copy_(src))
    return 2 * n / (ms * 1e-3) / 1e9


def _pct(xs, p):
    s = sorted(xs)
    return s[min(len(s) - 1, int(round(p / 100.0 * (len(s) - 1))))]


def _base(args, metric, value, unit, ms, cfg, dtype="bf16"):
    return {"metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype,
            "data": "synthetic: N(0,1) q/k/v rounded to bf16 (seeded per frame)", "config": cfg}


def _mfma_roofline(flops, ms, traffic=None):
    tf = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic}


def _hbm_pass(nbytes, ms, ceiling_gbs):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel_us": round(ms * 1e3, 2), "bytes": nbytes, "GBps": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "copy_ceiling_GBps": round(ceiling_gbs, 1),
            "frac_of_copy_ceiling": round(gbs / ceiling_gbs, 4)}


def _dev(torch, arrs):
    return tuple(torch.from_numpy(x).to("cuda").to(torch.bfloat16) for x in arrs)


def _cores():
    return len(os.sched_getaffinity(0))


def _cpu(value, unit, sample):
    return {"value": round(value, 6), "unit": unit, "cores": _cores(), "kind": "oracle", "sample": sample}


# The attention kernel's sources and its compile flags: a traffic summary
# under profiles/ applies while their hash matches.
KERNEL_SOURCES = ("sliding_window_kv_amd/csrc/attn_kernels.hip", "sliding_window_kv_amd/csrc/kernels_common.hpp",
                  "sliding_window_kv_amd/csrc/launch.hpp")


def _sources_sha256(paths):
    import hashlib
    from sliding_window_kv_amd import build as B
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    flags = B.COMMON + B.DEVICE_FLAGS + B.PER_SOURCE_FLAGS.get("attn_kernels.hip", [])
    h.update(" ".join(x.replace(ROOT, "<repo>") for x in flags).encode())
    return h.hexdigest()


def _measured_traffic(workload):
    """HBM bytes per attention launch of a workload from its committed
    counter summary, or None when the kernel sources no longer match."""
    path = os.path.join(ROOT, "profiles", f"attention_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("kernel_sources_sha256") != _sources_sha256(KERNEL_SOURCES):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _oracle_stream_rate(make_cache, frames, warm, steps, flops_of, budget_s=12.0):
    """Oracle seconds over `steps` steady steps after `warm` untimed ones
    (at most about budget_s of timed work); returns (TFLOP/s, steps, seconds)."""
    oc, step = make_cache()
    for t in range(warm):
        step(oc, t, frames(t), False)
    dt, n, fl = 0.0, 0, 0.0
    for t in range(warm, warm + steps):
        f = frames(t)
        t0 = time.perf_counter()
        keys = step(oc, t, f, True)
        dt += time.perf_counter() - t0
        fl += flops_of(keys)
        n += 1
        if dt > budget_s:
            break
    return fl / dt / 1e12, n, dt


# ---------------------------------------------------------------------------
# single streaming step (headline)
# ---------------------------------------------------------------------------

def bench_stream(args, torch, swa):
    from swa_synth import frame_qkv
    P, H, D, W, S = 1374, 16, 64, 16, 8
    cache = swa.SwaCache(swa.make_config(P, H, D, sliding_window_size=W, scale_frames=S))
    if args.splits is not None:
        cache.set_splits(args.splits)
    npool = 97
    pool = [_dev(torch, frame_qkv(2, i, P, H, D)) for i in range(npool)]
    out = torch.empty((P, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, P), dtype=torch.float32, device="cuda")
    state = {"t": 0}

    def step(_):
        t = state["t"]
        q, k, v = pool[t % npool]
        cache.step(0, t, q, k, v, True, out, None)
        state["t"] = t + 1

    for _ in range(S + W + args.warmup):        # fill the window, then warm up
        step(0)
    keys = sum(p[4] for p in cache.pages())
    assert keys == (S + W) * P
    flops = 4.0 * D * H * P * keys
    ms_step = _timed(torch, step, args.steps)
    q0 = pool[0][0]
    ms_attn = _timed(torch, lambda _: cache.attend(0, q0, out, None), args.steps)
    ms_attn_lse = _timed(torch, lambda _: cache.attend(0, q0, out, lse), args.steps)

    def app(_):
        t = state["t"]
        cache.append(0, t, pool[t % npool][1], pool[t % npool][2], True)
        cache.evict(0)
        state["t"] = t + 1

    append_bytes = 2 * 2 * P * H * D * 2
    ms_app = _device_ms(torch, app)
    # The same attention call over a cache filled with zero frames and a zero
    # query: the same kernel and instruction stream (every score 0, every
    # probability 1), but the matrix and vector units switch far fewer bits.
    # Timed last, so its launches are the last attention dispatches of the run.
    zcache = swa.SwaCache(swa.make_config(P, H, D, sliding_window_size=W, scale_frames=S))
    if args.splits is not None:
        zcache.set_splits(args.splits)
    zero = torch.zeros((P, H, D), dtype=torch.bfloat16, device="cuda")
    for t in range(S + W + 1):
        zcache.step(0, t, zero, zero, zero, True, out, None)
    ms_attn_zero = _timed(torch, lambda _: zcache.attend(0, zero, out, None), args.steps)
    del zcache
    res = _base(args, METRIC, flops / (ms_step * 1e-3) / 1e12, "TFLOP/s", ms_step,
                {"workload": "stream_step", "tokens_per_frame": P, "heads": H, "head_dim": D, "scale_frames": S,
                 "window_frames": W, "visible_keys": keys, "splits": args.splits or "auto", "lse_output": False})
    res.update({
        "frames_per_s_per_layer": round(1000.0 / ms_step, 1),
        "attention_ms": round(ms_attn, 5),
        "attention_with_lse_ms": round(ms_attn_lse, 5),
        "attention_ms_zero_inputs": round(ms_attn_zero, 5),
        "roofline": _mfma_roofline(flops, ms_attn, _measured_traffic("stream")),
        "append": _hbm_pass(append_bytes, ms_app, _copy_ceiling_gbs(torch, append_bytes)),
    })
    if not args.no_cpu:
        from oracle import CacheConfig, NaiveRingCache

        def make():
            def st(oc, t, f, timed):
                q, k, v = f
                oc.append(t, k, v, True)
                oc.evict()
                if timed:
                    oc.attend(q)
                return sum(p[4] for p in oc.visible_pages())
            return NaiveRingCache(CacheConfig(P=P, sliding_window_size=W, scale_frames=S)), st

        tf, n, dt = _oracle_stream_rate(make, lambda t: frame_qkv(2, t, P, H, D), S + W, 8,
                                        lambda keys: 4.0 * D * H * P * keys, budget_s=10.0)
        res["cpu_baseline"] = _cpu(tf, "TFLOP/s", f"{n} steady-state steps (append, evict, attend over {keys} keys "
                                                  f"each), {dt:.2f} s in float64 NumPy")
    return res


# ---------------------------------------------------------------------------
# tiny fp32 workload (latency-bound)
# ---------------------------------------------------------------------------

def bench_tiny(args, torch, swa):
    import numpy as np
    from swa_synth import chunk_qkv
    F, P, H, D, W, S = 6, 21, 2, 32, 2, 1
    qn, kn, vn = chunk_qkv(1, F, P, H, D, bf16=False)
    q, k, v = (torch.from_numpy(x).to("cuda") for x in (qn, kn, vn))
    out = torch.empty_like(q)
    ws = torch.empty(swa.swa_prefill_workspace_bytes(F, P, H, D, swa.SWA_F32), dtype=torch.uint8, device="cuda")
    pairs = sum(1 for i in range(F) for j in range(i + 1) if j >= i - W + 1 or j < S)
    flops = 4.0 * D * H * P * P * pairs
    for _ in range(args.warmup):
        swa.prefill_t(q, k, v, F, P, W, 1, S, out, None, ws)
    ms_pre = _device_ms(torch, lambda _: swa.prefill_t(q, k, v, F, P, W, 1, S, out, None, ws))
    cache = swa.SwaCache(swa.make_config(P, H, D, dtype=swa.SWA_F32, sliding_window_size=W, scale_frames=S))
    outs = torch.empty((P, H, D), dtype=torch.float32, device="cuda")
    frames = [tuple(x[t * P:(t + 1) * P] for x in (q, k, v)) for t in range(F)]

    def replay(_):
        cache.reset()
        for t in range(F):
            cache.step(0, t, *frames[t], True, outs, None)

    replay(0)
    ms_replay = _timed(torch, replay, max(1, args.steps // 4))
    res = _base(args, "tiny fp32 masked prefill, TFLOP/s (6 frames x 21 tokens, window 2, 1 scale frame)",
                flops / (ms_pre * 1e-3) / 1e12, "TFLOP/s", ms_pre,
                {"workload": "tiny_fp32", "frames": F, "tokens_per_frame": P, "heads": H, "head_dim": D,
                 "window_frames": W, "scale_frames": S, "visible_frame_pairs": pairs}, dtype="fp32")
    res["data"] = "synthetic: N(0,1) q/k/v float32 (seeded per frame)"
    tf = flops / (ms_pre * 1e-3) / 1e12
    res["roofline"] = {"bound": "alu", "achieved": round(tf, 4), "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": round(tf / FP32_VECTOR_PEAK_TFLOPS, 6), "traffic": None,
                       "note": "latency-bound: 1.69 MFLOP per call; the prefill call is two launches"}
    res["prefill_us"] = round(ms_pre * 1e3, 2)
    res["stream_replay_us_per_frame"] = round(ms_replay * 1e3 / F, 2)
    if not args.no_cpu:
        from oracle import CacheConfig, prefill, stream_replay
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 2.0:
            prefill(qn, kn, vn, F, P, W, 1, S)
            reps += 1
        dt = time.perf_counter() - t0
        t1 = time.perf_counter()
        for _ in stream_replay(CacheConfig(P=P, sliding_window_size=W, scale_frames=S),
                               lambda t: tuple(x[t * P:(t + 1) * P] for x in (qn, kn, vn)), F):
            pass
        dt_replay = time.perf_counter() - t1
        res["cpu_baseline"] = _cpu(reps * flops / dt / 1e12, "TFLOP/s",
                                   f"{reps} full prefills in {dt:.2f} s (oracle stream replay of the 6 frames: "
                                   f"{dt_replay * 1e3:.1f} ms)")
    return res


# ---------------------------------------------------------------------------
# chunked masked prefill
# ---------------------------------------------------------------------------

def bench_prefill(args, torch, swa):
    import numpy as np
    from swa_synth import chunk_qkv
    F, P, H, D, W, S = 32, 1374, 16, 64, 8, 8
    qn, kn, vn = chunk_qkv(3, F, P, H, D)
    q, k, v = _dev(torch, (qn, kn, vn))
    out = torch.empty_like(q)
    need = swa.swa_prefill_workspace_bytes(F, P, H, D, swa.SWA_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    # visible (query frame, key frame) pairs: j <= i and (j >= i - W + 1 or j < S)
    pairs = sum(1 for i in range(F) for j in range(i + 1) if j >= i - W + 1 or j < S)
    flops = 4.0 * D * H * P * P * pairs
    for _ in range(args.warmup):
        swa.prefill_t(q, k, v, F, P, W, 1, S, out, None, ws)
    ms = _timed(torch, lambda _: swa.prefill_t(q, k, v, F, P, W, 1, S, out, None, ws), max(1, args.steps // 10))
    res = _base(args, "prefill attention TFLOP/s (32 frames x 1374 tokens, window 8, 8 scale frames)",
                flops / (ms * 1e-3) / 1e12, "TFLOP/s", ms,
                {"workload": "chunked_prefill", "frames": F, "tokens_per_frame": P, "heads": H, "head_dim": D,
                 "window_frames": W, "scale_frames": S, "visible_frame_pairs": pairs, "lse_output": False})
    res["frames_per_s_per_layer"] = round(F * 1000.0 / ms, 1)
    # the call is the chunk layout (K rows and V^T of all 32 frames into the
    # workspace) followed by the attention: the roofline charges the whole
    # call to the attention, a lower bound on the attention kernel alone
    res["roofline"] = _mfma_roofline(flops, ms, _measured_traffic("prefill"))
    res["roofline"]["note"] = "whole prefill call (chunk layout + attention) against the attention FLOPs"
    chunk_bytes = 2 * 2 * F * P * H * D * 2
    res["chunk_layout_bytes"] = chunk_bytes
    res["copy_ceiling_GBps_at_chunk_size"] = round(_copy_ceiling_gbs(torch, chunk_bytes), 1)
    if not args.no_cpu:
        # oracle rows of query frames 0, 16 and 31 (1, 16 and 16 visible frames)
        from oracle import frame_visibility, masked_attention
        vis = frame_visibility(F, W, 1, S)
        assert int(vis.sum()) == pairs
        fk = np.arange(F * P) // P
        t0 = time.perf_counter()
        sample_pairs = 0
        for i in (0, 16, 31):
            rows = slice(i * P, (i + 1) * P)
            mask = np.broadcast_to(vis[i][fk][None, :], (P, F * P))
            masked_attention(qn[rows], kn, vn, mask)
            sample_pairs += int(vis[i].sum())
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = _cpu(4.0 * D * H * P * P * sample_pairs / dt / 1e12, "TFLOP/s",
                                   f"query frames 0, 16, 31 ({sample_pairs} frame pairs), {dt:.2f} s")
    return res


# ---------------------------------------------------------------------------
# long stream with 3-D RoPE
# ---------------------------------------------------------------------------

def bench_rope(args, torch, swa):
    import numpy as np
    from swa_synth import frame_positions, frame_qkv
    P, H, D, S = 1374, 16, 64, 8
    sws, nfpb, T = 6, 4, 2000
    W = sws * nfpb
    bands = (12, 10, 10)
    cache = swa.SwaCache(swa.make_config(P, H, D, sliding_window_size=sws, num_frame_per_block=nfpb,
                                         scale_frames=S, rope=bands, rope_theta=10000.0))
    if args.splits is not None:
        cache.set_splits(args.splits)
    npool = 97
    pool = [_dev(torch, frame_qkv(4, i, P, H, D)) for i in range(npool)]
    pos = torch.from_numpy(np.stack([frame_positions(t, 37, 37, 5) for t in range(T)])).to("cuda")
    out = torch.empty((P, H, D), dtype=torch.bfloat16, device="cuda")

    def step(t):
        # the fused RoPE rotates the pool's q in place (a rotation: the inputs
        # stay N(0,1) for timing purposes)
        q, k, v = pool[t % npool]
        cache.step(0, t, q, k, v, True, out, None, pos=pos[t])

    t0 = S + W - 1                               # 31: cache full from here on
    for t in range(t0):
        step(t)
    times = _per_step(torch, step, list(range(t0, T)))
    ms = sum(times) / len(times)
    keys = (S + W) * P
    flops = 4.0 * D * H * P * keys
    ms_attn = _timed(torch, lambda _: cache.attend(0, pool[0][0], out, None), max(args.steps, 1))
    res = _base(args, "streaming step with 3-D RoPE, TFLOP/s (1374 q x 43,968 keys)",
                flops / (ms * 1e-3) / 1e12, "TFLOP/s", ms,
                {"workload": "rope_stream", "frames": T, "tokens_per_frame": P, "heads": H, "head_dim": D,
                 "window_frames": W, "scale_frames": S, "rope_pairs": list(bands), "visible_keys": keys,
                 "timed_steps": f"t in [{t0}, {T})", "lse_output": False})
    res["steps"] = len(times)
    res["warmup"] = t0
    res["frames_per_s_per_layer"] = round(1000.0 / ms, 1)
    res["p50_ms"] = round(_pct(times, 50), 5)
    res["p99_ms"] = round(_pct(times, 99), 5)
    res["attention_ms"] = round(ms_attn, 5)
    res["roofline"] = _mfma_roofline(flops, ms_attn, _measured_traffic("rope"))
    # the standalone 3-D RoPE pass (rope3d_apply on q and k in place):
    # 4 x P x H x D x 2 B moved plus the positions; its device time per launch
    qr, kr = pool[0][0].clone(), pool[0][1].clone()
    rope_bytes = 4 * P * H * D * 2 + 12 * P
    ms_rope = _device_ms(torch, lambda i: swa.rope3d_t(qr, kr, pos[i % T], bands))
    res["rope_standalone"] = _hbm_pass(rope_bytes, ms_rope, _copy_ceiling_gbs(torch, rope_bytes))
    # the step minus its attention call: the fused RoPE + append pass, plus
    # host bookkeeping and launch gaps (kernel time alone: profiles/)
    res["rope_append_fused_bytes"] = 6 * P * H * D * 2
    res["copy_ceiling_GBps_at_fused_size"] = round(_copy_ceiling_gbs(torch, 6 * P * H * D * 2), 1)
    res["step_minus_attention_us"] = round((ms - ms_attn) * 1e3, 2)
    if not args.no_cpu:
        from oracle import CacheConfig, NaiveRingCache, rope3d

        def make():
            def st(oc, t, f, timed):
                q, k, v = f
                pt = frame_positions(t, 37, 37, 5)
                kr_ = rope3d(k, pt, *bands)
                oc.append(t, kr_, v, True)
                oc.evict()
                if timed:
                    oc.attend(rope3d(q, pt, *bands))
                return sum(p[4] for p in oc.visible_pages())
            return NaiveRingCache(CacheConfig(P=P, sliding_window_size=sws, num_frame_per_block=nfpb,
                                              scale_frames=S)), st

        tf, n, dt = _oracle_stream_rate(make, lambda t: frame_qkv(4, t % npool, P, H, D), t0, 6,
                                        lambda keys: 4.0 * D * H * P * keys)
        res["cpu_baseline"] = _cpu(tf, "TFLOP/s", f"{n} steady-state steps from t = {t0} (rope, append, evict, "
                                                  f"attend over {keys} keys each), {dt:.2f} s in float64 NumPy")
    return res


# ---------------------------------------------------------------------------
# the RoPE stream with the per-head q/k norm fused into the append pass
# ---------------------------------------------------------------------------

def bench_normed(args, torch, swa):
    import numpy as np
    from swa_synth import frame_positions, frame_qkv, norm_weights
    P, H, D, S = 1374, 16, 64, 8
    sws, nfpb = 6, 4
    W = sws * nfpb
    t0, T = S + W - 1, S + W - 1 + max(args.steps, 1)
    cfg = swa.make_config(P, H, D, sliding_window_size=sws, num_frame_per_block=nfpb, scale_frames=S,
                          rope=(12, 10, 10), rope_theta=10000.0)
    fused, split = swa.SwaCache(cfg), swa.SwaCache(cfg)
    if args.splits is not None:
        fused.set_splits(args.splits)
        split.set_splits(args.splits)
    npool = 97
    pool = [_dev(torch, frame_qkv(6, i, P, H, D)) for i in range(npool)]
    pos = torch.from_numpy(np.stack([frame_positions(t, 37, 37, 5) for t in range(T)])).to("cuda")
    w = torch.from_numpy(norm_weights(6, D)).to("cuda")
    out = torch.empty((P, H, D), dtype=torch.bfloat16, device="cuda")

    # both variants normalise and rotate the pool's q (and the separate norm
    # pass its k) in place: for timing only
    def step_fused(t):
        q, k, v = pool[t % npool]
        fused.step_normed(0, t, q, k, v, w, 1e-5, True, out, None, pos=pos[t])

    def step_split(t):
        q, k, v = pool[t % npool]
        swa.qk_norm_t(q, k, w, 1e-5)
        split.step(0, t, q, k, v, True, out, None, pos=pos[t])

    for t in range(t0):
        step_fused(t)
        step_split(t)
    tf = _per_step(torch, step_fused, list(range(t0, T)))
    ts = _per_step(torch, step_split, list(range(t0, T)))
    ms, ms_split = sum(tf) / len(tf), sum(ts) / len(ts)
    keys = (S + W) * P
    flops = 4.0 * D * H * P * keys
    ms_attn = _timed(torch, lambda _: fused.attend(0, pool[0][0], out, None), max(args.steps, 1))
    qn, kn = pool[1][0].clone(), pool[1][1].clone()
    ms_norm = _device_ms(torch, lambda _: swa.qk_norm_t(qn, kn, w, 1e-5))
    res = _base(args, "streaming step with fused q/k norm + 3-D RoPE + append, TFLOP/s (1374 q x 43,968 keys)",
                flops / (ms * 1e-3) / 1e12, "TFLOP/s", ms,
                {"workload": "normed_rope_stream", "tokens_per_frame": P, "heads": H, "head_dim": D,
                 "window_frames": W, "scale_frames": S, "rope_pairs": [12, 10, 10], "visible_keys": keys,
                 "norm": "per-head layer norm, eps 1e-5", "timed_steps": f"t in [{t0}, {T})", "lse_output": False})
    res["steps"] = len(tf)
    res["warmup"] = t0
    res["frames_per_s_per_layer"] = round(1000.0 / ms, 1)
    res["separate_passes_ms_per_step"] = round(ms_split, 5)
    res["attention_ms"] = round(ms_attn, 5)
    res["roofline"] = _mfma_roofline(flops, ms_attn)
    norm_bytes = 4 * P * H * D * 2
    res["norm_standalone"] = _hbm_pass(norm_bytes, ms_norm, _copy_ceiling_gbs(torch, norm_bytes))
    res["fused_pre_attention_bytes"] = 6 * P * H * D * 2
    res["separate_pre_attention_bytes"] = 10 * P * H * D * 2
    if not args.no_cpu:
        from oracle import CacheConfig, NaiveRingCache, head_layer_norm, rope3d
        wn = norm_weights(6, D).astype(np.float64)

        def make():
            def st(oc, t, f, timed):
                q, k, v = f
                pt = frame_positions(t, 37, 37, 5)
                oc.append(t, rope3d(head_layer_norm(k, wn[2], wn[3]), pt, 12, 10, 10), v, True)
                oc.evict()
                if timed:
                    oc.attend(rope3d(head_layer_norm(q, wn[0], wn[1]), pt, 12, 10, 10))
                return sum(p[4] for p in oc.visible_pages())
            return NaiveRingCache(CacheConfig(P=P, sliding_window_size=sws, num_frame_per_block=nfpb,
                                              scale_frames=S)), st

        tf_cpu, n, dt = _oracle_stream_rate(make, lambda t: frame_qkv(6, t % npool, P, H, D), t0, 4,
                                            lambda keys: 4.0 * D * H * P * keys)
        res["cpu_baseline"] = _cpu(tf_cpu, "TFLOP/s", f"{n} steady-state steps (norm, rope, append, evict, attend "
                                                      f"over {keys} keys each), {dt:.2f} s in float64 NumPy")
    return res


# ---------------------------------------------------------------------------
# captured multi-layer step
# ---------------------------------------------------------------------------

def bench_graph(args, torch, swa):
    from swa_synth import frame_qkv
    L, P, H, D, W, S = 12, 1374, 16, 64, 16, 8
    cfg = swa.make_config(P, H, D, sliding_window_size=W, scale_frames=S, num_layers=L)
    gcache, ecache = swa.SwaCache(cfg), swa.SwaCache(cfg)
    if args.splits is not None:
        gcache.set_splits(args.splits)
        ecache.set_splits(args.splits)
    qkv = [_dev(torch, frame_qkv(9, l, P, H, D)) for l in range(L)]   # one frame per layer, re-appended each step
    outs = [torch.empty((P, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    graph = swa.SwaGraph(gcache, [x[0] for x in qkv], [x[1] for x in qkv], [x[2] for x in qkv], outs)
    state = {"g": 0, "e": 0}

    def step_graph(_):
        graph.step(state["g"], True)
        state["g"] += 1

    def step_eager(_):
        t = state["e"]
        for l in range(L):
            q, k, v = qkv[l]
            ecache.step(l, t, q, k, v, True, outs[l], None)
        state["e"] = t + 1

    for _ in range(S + W + args.warmup):
        step_graph(0)
        step_eager(0)
    keys = sum(p[4] for p in gcache.pages(0))
    assert keys == (S + W) * P
    flops = 4.0 * D * H * P * keys * L
    ms = _timed(torch, step_graph, args.steps)
    ms_eager = _timed(torch, step_eager, args.steps)

    def host_ms(fn, reps=15, n=3):
        """Host time to enqueue one step: median over bursts of n steps, each
        started on an idle GPU (the queue never fills)."""
        per = []
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                fn(0)
            per.append((time.perf_counter() - t0) / n * 1e3)
        torch.cuda.synchronize()
        return sorted(per)[len(per) // 2]

    host_graph, host_eager = host_ms(step_graph), host_ms(step_eager)
    graph.close()
    res = _base(args, f"captured {L}-layer streaming step, TFLOP/s (1374 q x 32,976 keys per layer)",
                flops / (ms * 1e-3) / 1e12, "TFLOP/s", ms,
                {"workload": "graph_step", "layers": L, "tokens_per_frame": P, "heads": H, "head_dim": D,
                 "scale_frames": S, "window_frames": W, "visible_keys": keys, "lse_output": False})
    res["frames_per_s_per_layer"] = round(1000.0 * L / ms, 1)
    res["eager_ms_per_step"] = round(ms_eager, 5)
    res["eager_frames_per_s_per_layer"] = round(1000.0 * L / ms_eager, 1)
    res["launches_per_step"] = {"captured": 2, "eager": 3 * L}
    res["host_enqueue_ms_per_step"] = {"captured": round(host_graph, 4), "eager": round(host_eager, 4)}
    res["roofline"] = _mfma_roofline(flops, ms)
    res["roofline"]["note"] = "whole captured step (12 x append, attention, merge) against the attention FLOPs"
    if not args.no_cpu:
        # layers are independent caches: the oracle steps one layer's cache
        # (the same frame re-appended every step, as in the captured step)
        from oracle import CacheConfig, NaiveRingCache

        def make():
            def st(oc, t, f, timed):
                q, k, v = f
                oc.append(t, k, v, True)
                oc.evict()
                if timed:
                    oc.attend(q)
                return sum(p[4] for p in oc.visible_pages())
            return NaiveRingCache(CacheConfig(P=P, sliding_window_size=W, scale_frames=S)), st

        frame0 = frame_qkv(9, 0, P, H, D)
        tf, n, dt = _oracle_stream_rate(make, lambda t: frame0, S + W, 8,
                                        lambda keys: 4.0 * D * H * P * keys, budget_s=10.0)
        res["cpu_baseline"] = _cpu(tf, "TFLOP/s", f"{n} steady-state layer steps of one layer's cache (append, evict, "
                                                  f"attend over {keys} keys each; the captured step runs {L} such "
                                                  f"layers), {dt:.2f} s in float64 NumPy")
    return res


# ---------------------------------------------------------------------------
# token-level decode over rolling buffers (grouped-query heads)
# ---------------------------------------------------------------------------

def bench_decode(args, torch, swa):
    from swa_synth import frame_qkv
    Hq, Hkv, W, D = 32, 8, 4096, 64
    res = None
    for B in (16, 1):
        dc = swa.DecodeCache(B, Hq, Hkv, W, D)
        npool = 61
        pool = []
        for i in range(npool):
            _, k, v = frame_qkv(7, i, B, Hkv, D)
            q = frame_qkv(1007, i, B, Hq, D)[0]
            pool.append(_dev(torch, (q, k, v)))
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")

        def step(pos):
            q, k, v = pool[pos % npool]
            dc.step(pos, q, k, v, out)

        for pos in range(W + args.warmup):           # fill the buffer, then warm up
            step(pos)
        t0 = W + args.warmup
        ms = _timed(torch, lambda i: step(t0 + i), args.steps)
        kv_bytes = 2 * B * Hkv * W * D * 2
        io_bytes = (2 * B * Hq * D + 2 * B * Hkv * D) * 2
        gbs = (kv_bytes + io_bytes) / (ms * 1e-3) / 1e9
        if res is None:
            res = _base(args, "token decode over a 4096-slot rolling buffer, GB/s of HBM (K, V, q, out)",
                        gbs, "GB/s", ms,
                        {"workload": "decode_gqa", "batch": B, "q_heads": Hq, "kv_heads": Hkv, "window": W,
                         "head_dim": D, "timed_positions": f"{t0} .. {t0 + args.steps - 1} (buffer full)"})
            res["tokens_per_s"] = round(B / (ms * 1e-3), 1)
            res["bytes_per_step"] = kv_bytes + io_bytes
            res["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                               "copy_ceiling_GBps": round(_copy_ceiling_gbs(torch, kv_bytes), 1),
                               "note": "whole step (attention with the new token's write, merge)"}
            if not args.no_cpu:
                from oracle import RollingDecodeCache
                oc = [RollingDecodeCache(W, Hkv, D) for _ in range(B)]
                toks = [(frame_qkv(1007, i, B, Hq, D)[0], *frame_qkv(7, i, B, Hkv, D)[1:]) for i in range(npool)]
                for pos in range(W):
                    _, k, v = toks[pos % npool]
                    for b in range(B):
                        oc[b].append(pos, k[b], v[b])
                t1 = time.perf_counter()
                n = 0
                while time.perf_counter() - t1 < 5.0:
                    q, k, v = toks[(W + n) % npool]
                    for b in range(B):
                        oc[b].append(W + n, k[b], v[b])
                        oc[b].attend(W + n, q[b])
                    n += 1
                dt = time.perf_counter() - t1
                res["cpu_baseline"] = _cpu(n * (kv_bytes + io_bytes) / dt / 1e9, "GB/s",
                                           f"{n} steady decode steps of batch {B} (append + attend per sequence), "
                                           f"{dt:.2f} s in float64 NumPy")
        else:
            res["batch1_ms_per_step"] = round(ms, 5)
            res["batch1_GBps"] = round(gbs, 1)
    return res


# ---------------------------------------------------------------------------
# ragged frames with retained specials and non-keyframes
# ---------------------------------------------------------------------------

def bench_specials(args, torch, swa):
    from swa_synth import frame_qkv
    P, H, D, W, S, ns, R, T = 1405, 16, 64, 16, 8, 5, 1000, 1600
    cache = swa.SwaCache(swa.make_config(P, H, D, sliding_window_size=W, scale_frames=S, cross_frame_special=True,
                                         special_row0=0, special_rows=ns, max_special_frames=R))
    if args.splits is not None:
        cache.set_splits(args.splits)
    npool = 97
    pool = [_dev(torch, frame_qkv(5, i, P, H, D)) for i in range(npool)]
    out = torch.empty((P, H, D), dtype=torch.bfloat16, device="cuda")
    key_of = lambda t: t % 3 != 2          # noqa: E731

    def step(t):
        q, k, v = pool[t % npool]
        cache.step(0, t, q, k, v, key_of(t), out, None)

    t0 = 1534
    for t in range(t0):
        step(t)
    idx = list(range(t0, T))
    times = _per_step(torch, step, idx)
    kf = [ms for t, ms in zip(idx, times) if key_of(t)]
    nk = [ms for t, ms in zip(idx, times) if not key_of(t)]
    ms_k = sum(kf) / len(kf)
    ms_n = sum(nk) / len(nk)
    keys_k = (S + W) * P + R * ns
    keys_n = keys_k + P
    fl_k = 4.0 * D * H * P * keys_k
    fl_n = 4.0 * D * H * P * keys_n
    ms = sum(times) / len(times)
    ms_attn = _timed(torch, lambda _: cache.attend(0, pool[0][0], out, None), max(args.steps, 1))
    res = _base(args, "streaming step with retained specials, TFLOP/s (1405 q x 38,720 / 40,125 keys)",
                (fl_k * len(kf) + fl_n * len(nk)) / (sum(times) * 1e-3) / 1e12, "TFLOP/s", ms,
                {"workload": "ragged_specials_stream", "frames": T, "tokens_per_frame": P, "heads": H,
                 "head_dim": D, "window_frames": W, "scale_frames": S, "special_rows": ns,
                 "retained_special_frames": R, "nonkeyframe": "t % 3 == 2", "timed_steps": f"t in [{t0}, {T})",
                 "lse_output": False})
    res["steps"] = len(times)
    res["warmup"] = t0
    res["keyframe_ms"] = round(ms_k, 5)
    res["nonkeyframe_ms"] = round(ms_n, 5)
    res["keyframe_TFLOPs"] = round(fl_k / (ms_k * 1e-3) / 1e12, 2)
    res["nonkeyframe_TFLOPs"] = round(fl_n / (ms_n * 1e-3) / 1e12, 2)
    res["frames_per_s_per_layer"] = round(1000.0 / ms, 1)
    res["attention_ms"] = round(ms_attn, 5)
    res["roofline"] = _mfma_roofline(fl_k, ms_attn, _measured_traffic("specials"))
    res["roofline"]["note"] = "attention call over the keyframe state (38,720 keys)"
    # the visible-page list of the full ring (1,000 special entries) built on
    # the device and read back (builder kernel + copy + synchronize), and the
    # host ring bookkeeping of one keyframe step on a bookkeeping-only cache
    # (append plan + evict, ctypes calls included)
    lat = []
    for _ in range(20):
        t1 = time.perf_counter()
        recs, n = cache.device_pages(0)
        lat.append((time.perf_counter() - t1) * 1e3)
    assert recs == cache.pages(0)
    res["page_list_records"] = n
    res["device_page_list_ms"] = round(sorted(lat)[len(lat) // 2], 4)
    cfg = swa.make_config(P, H, D, sliding_window_size=W, scale_frames=S, cross_frame_special=True, special_row0=0,
                          special_rows=ns, max_special_frames=R)
    dry = swa.swa_cache_create(cfg, None, 0)
    for t in range(t0):
        swa.kvcache_append(dry, 0, t, None, None, True)
        swa.kvcache_evict(dry, 0)
    lat = []
    for t in range(t0, t0 + 200):
        t1 = time.perf_counter()
        swa.kvcache_append(dry, 0, t, None, None, True)
        swa.kvcache_evict(dry, 0)
        lat.append((time.perf_counter() - t1) * 1e6)
    swa.swa_cache_destroy(dry)
    res["host_bookkeeping_us_per_keyframe"] = round(sorted(lat)[len(lat) // 2], 2)
    if not args.no_cpu:
        from oracle import CacheConfig, NaiveRingCache

        def make():
            def st(oc, t, f, timed):
                q, k, v = f
                kf_ = key_of(t)
                oc.append(t, k, v, kf_)
                if kf_:
                    oc.evict()
                keys = sum(p[4] for p in oc.visible_pages())
                if timed:
                    oc.attend(q)
                if not kf_:
                    oc.rollback()
                return keys
            return NaiveRingCache(CacheConfig(P=P, sliding_window_size=W, scale_frames=S, cross_frame_special=True,
                                              special_row0=0, special_rows=ns, max_special_frames=R)), st

        host_pool = {}

        def frames(t):
            if t % npool not in host_pool:
                host_pool[t % npool] = frame_qkv(5, t % npool, P, H, D)
            return host_pool[t % npool]

        tf, n, dt = _oracle_stream_rate(make, frames, t0, 6, lambda keys: 4.0 * D * H * P * keys)
        res["cpu_baseline"] = _cpu(tf, "TFLOP/s", f"{n} steady steps from t = {t0} (keyframes and a non-keyframe, "
                                                  f"about 39k keys each), {dt:.2f} s in float64 NumPy")
    return res


WORKLOADS = {"stream": bench_stream, "tiny": bench_tiny, "prefill": bench_prefill, "rope": bench_rope,
             "specials": bench_specials, "normed": bench_normed, "decode": bench_decode, "graph": bench_graph}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="stream", choices=list(WORKLOADS) + ["all"])
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: use --gpus 1 (a multi-GPU, head-sharded layout is not implemented)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import sliding_window_kv_amd as swa
    swa.lib()
    torch.cuda.set_device(0)
    order = list(WORKLOADS) if args.workload == "all" else [args.workload]
    for w in order:
        print(json.dumps(WORKLOADS[w](args, torch, swa)), flush=True)


if __name__ == "__main__":
    main()
