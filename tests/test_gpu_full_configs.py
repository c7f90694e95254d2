"""GPU parity at the stated sizes of the long-stream workloads, and a
key-inclusion closed form at full size (MI355X only).

  * RoPE stream: 2000 frames of P = 1374 (37 x 37 patches + 5 special
    tokens), H = 16, D = 64, window 6 blocks x 4 frames = 24 frames, 8 scale
    frames, 3-D RoPE theta 1e4 on 12 / 10 / 10 pairs from (t, row, col).
  * Specials stream: 1600 frames of P = 1405 (28 x 50 + 5), window 16
    frames, 8 scale frames, 5 special rows of up to 1000 evicted frames
    retained, frame t a non-keyframe iff t mod 3 == 2.

Every step runs through the C ABI in the bench's launch configuration
(automatic work split).  The host and the device page lists are compared
bit-exact with the oracle at every step.  Outputs and LSE are compared at
the steps [0, 40], every multiple of 97 and the last steps (the specials
stream also at [1534, 1540], where its special ring has filled), on sampled
query rows and heads (attention heads are independent): the oracle
(stream_replay) runs on those heads only.
"""
import math

import numpy as np
import pytest
import torch

import sliding_window_kv_amd as swa
from gpu_helpers import assert_close_bf16, bf16_round_f64, case, dev, host, lse_tol, ulp_bf16
from oracle import CacheConfig, NaiveRingCache, stream_replay
from swa_synth import frame_positions, frame_qkv

pytestmark = pytest.mark.gpu

ROWS = np.array([0, 1, 4, 5, 63, 64, 127, 128, 700, 1279, 1280, 1300, 1343, 1344, 1373])
HEADS = np.array([0, 7, 15])
NPOOL = 97


def _pool(cfg_id, P, H, D):
    """Frames 0..NPOOL-1 on the device (all heads) and on the host (sampled heads)."""
    devf, hostf = [], []
    for i in range(NPOOL):
        q, k, v = frame_qkv(cfg_id, i, P, H, D)
        devf.append((dev(q), dev(k), dev(v)))
        hostf.append((q[:, HEADS], k[:, HEADS], v[:, HEADS]))
    return devf, hostf


def _check_step(gc, t, pages, ro, rl, out, lse, n_keys, worst, keyframe=True):
    # `pages` are the records the step attended over; after a non-keyframe's
    # step the library has rolled it back, and the pending frame is the last
    # record (ascending frame order)
    after = pages
    if not keyframe:
        assert pages[-1][0] == t and pages[-1][2] == gc.layout.scratch_slot
        after = pages[:-1]
    assert gc.pages() == after, f"host pages t={t}"
    dp, n = gc.device_pages(cap=len(after) + 1)
    assert n == len(after) and dp == after, f"device pages t={t}"
    if ro is None:
        return
    got = host(out)[ROWS][:, HEADS]
    mx, mean = assert_close_bf16(got, ro, f"out t={t}")
    gl = host(lse)[HEADS][:, ROWS]
    le = float(np.abs(gl - rl).max())
    assert le <= lse_tol(n_keys), f"lse t={t}: {le:.3e} > {lse_tol(n_keys):.3e}"
    worst[0] = max(worst[0], mx)
    worst[1] = max(worst[1], le / lse_tol(n_keys))


def test_rope_stream_2000_frames():
    P, H, D, sws, nfpb, S, T = 1374, 16, 64, 6, 4, 8, 2000
    bands = (12, 10, 10)
    case(f"RoPE stream: {T} frames, P={P}, H={H}, window {sws}x{nfpb}, S={S}, bands {bands}")
    record = set(range(41)) | set(range(0, T, NPOOL)) | set(range(T - 5, T))
    devf, hostf = _pool(4, P, H, D)
    gc = swa.SwaCache(swa.make_config(P, H, D, sliding_window_size=sws, num_frame_per_block=nfpb, scale_frames=S,
                                      rope=bands, rope_theta=10000.0))
    ocfg = CacheConfig(P=P, sliding_window_size=sws, num_frame_per_block=nfpb, scale_frames=S)
    pos_host = lambda t: frame_positions(t, 37, 37, 5)          # noqa: E731
    qbuf = torch.empty((P, H, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(qbuf)
    lse = torch.empty((H, P), dtype=torch.float32, device="cuda")
    worst = [0.0, 0.0]
    # the rotated q and k are held in bf16 (q in place, k in the cache): the
    # oracle rotates exactly, then rounds them the same way
    ref = stream_replay(ocfg, lambda t: hostf[t % NPOOL], T, pos_of=pos_host, rope_pairs=bands, record=record,
                        rows=ROWS, store=bf16_round_f64)
    for t, pages, ro, rl in ref:
        q, k, v = devf[t % NPOOL]
        qbuf.copy_(q)                        # the fused RoPE rotates q in place
        gc.step(0, t, qbuf, k, v, True, out, lse, pos=torch.from_numpy(pos_host(t)).cuda())
        _check_step(gc, t, pages, ro, rl, out, lse, sum(p[4] for p in pages), worst)
    print(f"worst max-abs {worst[0]:.3e}, worst lse error / tolerance {worst[1]:.3f}", flush=True)
    gc.close()


def test_specials_stream_1600_frames():
    P, H, D, W, S, ns, R, T = 1405, 16, 64, 16, 8, 5, 1000, 1600
    case(f"specials stream: {T} frames, P={P}, window {W}, S={S}, {ns} special rows x R={R}, t%3==2 non-key")
    key = lambda t: t % 3 != 2                                  # noqa: E731
    record = set(range(41)) | set(range(0, T, NPOOL)) | set(range(1534, 1541)) | set(range(T - 5, T))
    devf, hostf = _pool(5, P, H, D)
    gc = swa.SwaCache(swa.make_config(P, H, D, sliding_window_size=W, scale_frames=S, cross_frame_special=True,
                                      special_row0=0, special_rows=ns, max_special_frames=R))
    ocfg = CacheConfig(P=P, sliding_window_size=W, scale_frames=S, cross_frame_special=True, special_row0=0,
                       special_rows=ns, max_special_frames=R)
    out = torch.empty((P, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, P), dtype=torch.float32, device="cuda")
    worst = [0.0, 0.0]
    full_ring = False
    for t, pages, ro, rl in stream_replay(ocfg, lambda t: hostf[t % NPOOL], T, keyframe_of=key, record=record,
                                          rows=ROWS):
        q, k, v = devf[t % NPOOL]
        gc.step(0, t, q, k, v, key(t), out, lse)
        _check_step(gc, t, pages, ro, rl, out, lse, sum(p[4] for p in pages), worst, key(t))
        full_ring = full_ring or sum(1 for p in pages if p[1] == swa.SWA_REGION_SPECIAL) == R
    assert full_ring
    print(f"worst max-abs {worst[0]:.3e}, worst lse error / tolerance {worst[1]:.3f}", flush=True)
    gc.close()


# ---------------------------------------------------------------------------
# key inclusion at full size: q = 0 gives every visible key weight 1 / N
# ---------------------------------------------------------------------------

def _onehot_v(t, P, H, D):
    """v of frame t: channel t mod 32 set on every row, plus channel
    32 + (row // 64) mod 32 (the row's 64-row block within the frame)."""
    v = torch.zeros((P, H, D), dtype=torch.bfloat16, device="cuda")
    v[:, :, t % 32] = 1
    r = torch.arange(P, device="cuda")
    v[r, :, 32 + (r // 64) % 32] = 1
    return v


@pytest.mark.parametrize("shape", ["stream_step", "stream_step_no_lse", "rope_stream", "specials"])
def test_key_inclusion_full_size(shape):
    """With q = 0 every visible key has weight exactly 1 / N: the LSE is
    ln(N) and the output is the mean of v over the visible rows, computed
    exactly by the oracle from its page list.  v marks each row's frame
    (mod 32) and 64-row block, so a lost, doubled or misplaced key tile
    changes the result by several bf16 ulps (or the LSE by about 64 / N),
    which the sampled-row checks of random data cannot resolve."""
    H, D = 16, 64
    want_lse = shape != "stream_step_no_lse"      # without an LSE output the pre-scaled-Q path runs
    if shape.startswith("stream_step"):
        P, sws, nfpb, S, R, bands, T, check = 1374, 16, 1, 8, 0, None, 64, (40, 63)
    elif shape == "rope_stream":
        P, sws, nfpb, S, R, bands, T, check = 1374, 6, 4, 8, 0, (12, 10, 10), 96, (63, 95)
    else:
        P, sws, nfpb, S, R, bands, T, check = 1405, 16, 1, 8, 1000, None, 1540, (1536, 1537, 1538, 1539)
    cross = R > 0
    key = (lambda t: t % 3 != 2) if cross else (lambda t: True)
    case(f"key inclusion {shape}: P={P} window {sws}x{nfpb} S={S} R={R}, {T} frames")
    gc = swa.SwaCache(swa.make_config(P, H, D, sliding_window_size=sws, num_frame_per_block=nfpb, scale_frames=S,
                                      cross_frame_special=cross, special_rows=5, max_special_frames=max(R, 1),
                                      rope=bands or (0, 0, 0)))
    oc = NaiveRingCache(CacheConfig(P=P, sliding_window_size=sws, num_frame_per_block=nfpb, scale_frames=S,
                                    cross_frame_special=cross, special_rows=5, max_special_frames=max(R, 1)))
    q0 = torch.zeros((P, H, D), dtype=torch.bfloat16, device="cuda")
    ks = [dev(frame_qkv(30, i, P, H, D)[1]) for i in range(7)]
    out = torch.empty_like(q0)
    lse = torch.empty((H, P), dtype=torch.float32, device="cuda") if want_lse else None
    zero_k = np.zeros((P, 1, D))
    for t in range(T):
        v = _onehot_v(t, P, H, D)
        pos = torch.from_numpy(frame_positions(t, 37, 37, 5)).cuda() if bands else None
        gc.step(0, t, q0, ks[t % 7], v, key(t), out, lse, pos=pos)
        vh = v[:, :1].float().cpu().numpy().astype(np.float64)
        oc.append(t, zero_k, vh, key(t))
        if key(t):
            oc.evict()
        if t in check:
            pages = oc.visible_pages()
            # the library has already rolled a non-keyframe back: its pending
            # page is the oracle's last record
            assert gc.pages() == (pages if key(t) else pages[:-1])
            n = sum(p[4] for p in pages)
            ro, rl = oc.attend(np.zeros((1, 1, D)))
            assert abs(rl[0, 0] - math.log(n)) < 1e-12
            got = host(out)
            exact = np.broadcast_to(ro[0, 0], got.shape)
            err = np.abs(got - exact)
            bound = 0.5 * ulp_bf16(exact) + 2.0 ** -22 * np.abs(exact)
            assert np.all(err <= bound), f"t={t}: output off by {float((err / ulp_bf16(exact)).max()):.2f} ulp"
            if want_lse:
                gl = host(lse)
                assert np.abs(gl - math.log(n)).max() <= 1e-5, f"t={t}: lse {gl.min()}..{gl.max()} vs ln {n}"
            if cross and t >= 1536:
                assert sum(1 for p in pages if p[1] == swa.SWA_REGION_SPECIAL) == R
        if not key(t):
            oc.rollback()
    gc.close()
