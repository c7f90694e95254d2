"""Benchmark of the streaming step on one MI355X.

Default workload (one JSON line): the single streaming step -- P = 1374
tokens per frame (37x37 patches + 1 camera + 4 register), H = 16, D = 64,
bf16, 8 scale frames + a 16-frame window, so every step attends 1374
queries to 24 x 1374 = 32,976 keys.  One step = append (K,V into the ring
page) + evict + attention (+ split combine), all through the C ABI.

  value        attention TFLOP/s of the whole step: algorithmic attention
               FLOPs (4*D*H*sum of visible keys) / measured step time
  roofline     the attention kernel alone against the bf16 dense MFMA peak
  cpu_baseline the float64 oracle on the machine's host cores, one steady step

Other workloads (--workload prefill|rope|specials) print their own line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 (published)
HBM_PEAK_GBS = 8000.0


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _timed(fn, steps):
    """Average ms of fn() over `steps` calls, bracketed by synchronize."""
    import torch
    torch.cuda.synchronize()
    a, b = _events()
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def cpu_baseline_stream(P, H, D, W, S, frames_fn):
    """Oracle (float64 NumPy) time of one steady-state step."""
    import numpy as np
    from oracle import CacheConfig, NaiveRingCache
    c = NaiveRingCache(CacheConfig(P=P, sliding_window_size=W, scale_frames=S))
    for t in range(S + W):
        q, k, v = frames_fn(t)
        c.append(t, k, v, True)
        c.evict()
    t = S + W
    q, k, v = frames_fn(t)
    t0 = time.perf_counter()
    c.append(t, k, v, True)
    c.evict()
    _, _ = c.attend(q)
    dt = time.perf_counter() - t0
    keys = sum(p[4] for p in c.visible_pages())
    return dt, keys


def bench_stream(args, torch, swa):
    from swa_synth import frame_qkv
    P, H, D, W, S = 1374, 16, 64, 16, 8
    cfg = swa.make_config(P, H, D, sliding_window_size=W, scale_frames=S)
    cache = swa.SwaCache(cfg)
    if args.splits is not None:
        cache.set_splits(args.splits)
    npool = 97 if args.pool is None else args.pool
    pool = []
    for i in range(npool):
        q, k, v = frame_qkv(2, i, P, H, D)
        pool.append(tuple(torch.from_numpy(x).to("cuda").to(torch.bfloat16) for x in (q, k, v)))
    out = torch.empty((P, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, P), dtype=torch.float32, device="cuda")
    state = {"t": 0}

    def step(_):
        t = state["t"]
        q, k, v = pool[t % npool]
        cache.step(0, t, q, k, v, True, out, lse)
        state["t"] = t + 1

    # fill the window to the steady state (S + W cached frames), then warm up
    for _ in range(S + W):
        step(0)
    for _ in range(args.warmup):
        step(0)
    keys = sum(p[4] for p in cache.pages())
    assert keys == (S + W) * P
    flops = 4.0 * D * H * P * keys

    ms_step = _timed(step, args.steps)
    # attention alone (same visible set, no state change)
    q0 = pool[0][0]
    ms_attn = _timed(lambda _: cache.attend(0, q0, out, lse), args.steps)
    # append + evict alone
    ms_app = _timed(lambda _: (lambda t: (cache.append(0, t, pool[t % npool][1], pool[t % npool][2], True),
                                          cache.evict(0), state.__setitem__("t", t + 1)))(state["t"]), args.steps)
    append_bytes = 2 * 2 * P * H * D * 2
    res = {
        "metric": "attention TFLOP/s and frames/s per layer, streaming step (1374 q x ~33k keys)",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: N(0,1) q/k/v rounded to bf16, 97 distinct frames cycled",
        "config": {"workload": "stream_step", "tokens_per_frame": P, "heads": H, "head_dim": D,
                   "scale_frames": S, "window_frames": W, "visible_keys": keys, "splits": args.splits or "auto"},
        "frames_per_s_per_layer": round(1000.0 / ms_step, 1),
        "attention_ms": round(ms_attn, 4),
        "append_evict_ms": round(ms_app, 4),
        "append_GBps": round(append_bytes / (ms_app * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(flops / (ms_attn * 1e-3) / 1e12, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (ms_attn * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None},
    }
    if not args.no_cpu:
        import numpy as np
        cores = len(os.sched_getaffinity(0))
        dt, okeys = cpu_baseline_stream(P, H, D, W, S, lambda t: frame_qkv(2, t % npool, P, H, D))
        oflops = 4.0 * D * H * P * okeys
        res["cpu_baseline"] = {"value": round(oflops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
                               "kind": "oracle",
                               "sample": f"one steady-state step (append+evict+attend, {okeys} keys), "
                                         f"{dt:.1f} s, float64 NumPy"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="stream", choices=["stream"])
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--pool", type=int, default=None)
    ap.add_argument("--no-cpu", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import sliding_window_kv_amd as swa
    swa.lib()
    torch.cuda.set_device(0)
    res = bench_stream(args, torch, swa)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
