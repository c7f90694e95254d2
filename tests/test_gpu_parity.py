"""GPU parity of the HIP path against the float64 oracle (MI355X only).

Every call goes through the C ABI of libswa.so.  Tolerances: fp32 path
max-abs 1e-5; bf16 path max-abs 2e-2 and mean-abs 2e-3 on N(0,1) inputs;
page lists, masks and cache bytes bit-exact.
"""
import numpy as np
import pytest
import torch

import sliding_window_kv_amd as swa
from gpu_helpers import (assert_close_bf16, assert_close_f32, bf16_round_f64, case, dev, host, lse_tol, vt_keys)
from oracle import (CacheConfig, NaiveRingCache, frame_visibility, masked_attention, prefill, rope3d,
                    token_mask)
from swa_synth import chunk_qkv, frame_positions, frame_qkv

pytestmark = pytest.mark.gpu


def _cache(P, H, D, dtype, W, S, nfpb=1, cross=False, ns=5, R=1000, max_frames=64, rope=(0, 0, 0),
           num_layers=1, sr0=0):
    cfg = swa.make_config(P, H, D, dtype=dtype, sliding_window_size=W, num_frame_per_block=nfpb,
                          scale_frames=S, cross_frame_special=cross, special_row0=sr0, special_rows=ns,
                          max_special_frames=R, max_frames=max_frames, rope=rope, num_layers=num_layers)
    ocfg = CacheConfig(P=P, sliding_window_size=W, num_frame_per_block=nfpb, scale_frames=S,
                       cross_frame_special=cross, special_row0=sr0, special_rows=ns, max_special_frames=R,
                       max_frames=max_frames)
    return swa.SwaCache(cfg), NaiveRingCache(ocfg)


# ---------------------------------------------------------------------------
# tiny fp32 workload: 6 frames, P=21, H=2, D=32, window 2, 1 scale frame
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("W,S", [(2, 1), (-1, 0), (6, 0), (1, 0)])
def test_prefill_f32_tiny(W, S):
    F, P, H, D = 6, 21, 2, 32
    case(f"prefill fp32 F={F} P={P} H={H} D={D} W={W} S={S}")
    q, k, v = chunk_qkv(1, F, P, H, D, bf16=False)
    ro, rl = prefill(q, k, v, F, P, W, 1, S)
    out = torch.empty((F * P, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((H, F * P), dtype=torch.float32, device="cuda")
    swa.prefill_t(dev(q, torch.float32), dev(k, torch.float32), dev(v, torch.float32), F, P, W, 1, S, out, lse)
    assert_close_f32(host(out), ro, "out")
    assert_close_f32(host(lse), rl, "lse")


@pytest.mark.parametrize("W,S", [(2, 1), (-1, 0), (6, 0)])
def test_stream_f32_tiny(W, S):
    F, P, H, D = 6, 21, 2, 32
    case(f"stream fp32 F={F} P={P} H={H} D={D} W={W} S={S}")
    gc, oc = _cache(P, H, D, swa.SWA_F32, W, S, max_frames=8)
    q, k, v = chunk_qkv(1, F, P, H, D, bf16=False)
    po, pl = prefill(q, k, v, F, P, W, 1, S)
    for t in range(F):
        rows = slice(t * P, (t + 1) * P)
        qd, kd, vd = (dev(x[rows], torch.float32) for x in (q, k, v))
        out = torch.empty_like(qd)
        lse = torch.empty((H, P), dtype=torch.float32, device="cuda")
        gc.step(0, t, qd, kd, vd, True, out, lse)
        ro, rl, pages = oc.step(t, q[rows], k[rows], v[rows], True)
        assert_close_f32(host(out), ro, f"out t={t}")
        assert_close_f32(host(lse), rl, f"lse t={t}")
        # streaming step t equals row block t of the masked prefill
        assert_close_f32(host(out), po[rows], f"stream==prefill t={t}")
        assert gc.pages() == pages
        dpages, n = gc.device_pages()
        assert dpages == pages and n == len(pages)


# ---------------------------------------------------------------------------
# bf16 prefill over several tiles with ragged frames
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("F,P,H,D,W,nfpb,S", [
    (5, 77, 2, 64, 2, 1, 1),
    (7, 130, 3, 64, 2, 1, 2),
    (4, 200, 2, 32, -1, 1, 0),
    (6, 61, 2, 64, 1, 2, 1),
])
def test_prefill_bf16(F, P, H, D, W, nfpb, S):
    case(f"prefill bf16 F={F} P={P} H={H} D={D} W={W} nfpb={nfpb} S={S}")
    q, k, v = chunk_qkv(3, F, P, H, D)
    ro, rl = prefill(q, k, v, F, P, W, nfpb, S)
    out = torch.empty((F * P, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, F * P), dtype=torch.float32, device="cuda")
    swa.prefill_t(dev(q), dev(k), dev(v), F, P, W, nfpb, S, out, lse)
    assert_close_bf16(host(out), ro, "out")
    keys = frame_visibility(F, W, nfpb, S).sum(axis=1) * P          # visible keys of each query frame
    tol = np.array([lse_tol(n) for n in keys]).repeat(P)[None, :]
    assert np.all(np.abs(host(lse) - rl) <= tol)


def test_prefill_mask_export_bit_exact():
    for (F, P, W, nfpb, S) in [(10, 3, 4, 1, 0), (12, 2, 2, 3, 2), (7, 5, -1, 1, 0), (32, 1, 8, 1, 8)]:
        case(f"mask F={F} P={P} W={W} nfpb={nfpb} S={S}")
        fr = torch.empty((F, F), dtype=torch.uint8, device="cuda")
        swa.prefill_mask_t(F, P, W, nfpb, S, False, fr)
        assert np.array_equal(host(fr).astype(bool), frame_visibility(F, W, nfpb, S))
        tok = torch.empty((F * P, F * P), dtype=torch.uint8, device="cuda")
        swa.prefill_mask_t(F, P, W, nfpb, S, True, tok)
        assert np.array_equal(host(tok).astype(bool), token_mask(F, P, W, nfpb, S))


# ---------------------------------------------------------------------------
# bf16 streaming with scale frames, retained specials and non-keyframes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("splits,S,ns", [(1, 2, 5), (3, 2, 5), (0, 2, 5), (0, 0, 5), (0, 2, 1)])
def test_stream_bf16_specials_nonkey(splits, S, ns):
    # S = 0 is include_scale_frames = false; ns = 1 is camera-only retention
    P, H, D, W, R = 45, 2, 64, 3, 4
    case(f"stream bf16 P={P} W={W} S={S} ns={ns} R={R} splits={splits}")
    gc, oc = _cache(P, H, D, swa.SWA_BF16, W, S, cross=True, ns=ns, R=R)
    gc.set_splits(splits)
    for t in range(18):
        kf = t % 3 != 2
        q, k, v = frame_qkv(5, t, P, H, D)
        qd, kd, vd = dev(q), dev(k), dev(v)
        out = torch.empty_like(qd)
        lse = torch.empty((H, P), dtype=torch.float32, device="cuda")
        gc.step(0, t, qd, kd, vd, kf, out, lse)
        ro, rl, pages = oc.step(t, q, k, v, kf)
        assert_close_bf16(host(out), ro, f"out t={t}")
        assert np.abs(host(lse) - rl).max() <= lse_tol(sum(p[4] for p in pages))
        assert gc.pages() == oc.visible_pages()
        # the device builder's list, on keyframes and on the pending
        # non-keyframe's step (kvcache_read_device_pages after the step's
        # rollback lists the cache without it)
        assert gc.device_pages()[0] == oc.visible_pages()


def test_cache_bytes_bit_exact():
    # K rows and transposed V rows of every visible frame page and special
    # entry equal the appended bf16 values exactly.
    P, H, D, W, S, ns, R = 37, 2, 64, 2, 1, 3, 2
    case(f"cache bytes P={P} W={W} S={S}")
    gc, oc = _cache(P, H, D, swa.SWA_BF16, W, S, cross=True, ns=ns, R=R)
    frames = {}
    for t in range(9):
        q, k, v = frame_qkv(6, t, P, H, D)
        frames[t] = (k, v)
        gc.append(0, t, dev(k), dev(v), True)
        gc.evict(0)
    torch.cuda.synchronize()
    kr, vr = gc.region_views(0)
    K = kr.float().cpu().numpy()
    V = vt_keys(vr.float().cpu().numpy())
    L = gc.layout
    for (f, region, slot, row0, nrows) in gc.pages():
        k, v = frames[f]
        if region == swa.SWA_REGION_FRAME:
            base = slot * P
            assert np.array_equal(K[:, base:base + P, :], k.transpose(1, 0, 2))
            assert np.array_equal(V[:, :, base:base + P], v.transpose(1, 2, 0))
        else:
            base = L.special_row_base + row0
            assert np.array_equal(K[:, base:base + nrows, :], k[:nrows].transpose(1, 0, 2))
            assert np.array_equal(V[:, :, base:base + nrows], v[:nrows].transpose(1, 2, 0))


@pytest.mark.parametrize("sr0", [0, 17])
def test_stream_f32_specials_nonkey(sr0):
    # fp32 cache: special-row retention inside the fp32 append, non-keyframes
    P, H, D, W, S, ns, R = 21, 2, 32, 2, 1, 3, 2
    case(f"stream fp32 specials P={P} W={W} S={S} ns={ns} R={R} rows from {sr0}")
    gc, oc = _cache(P, H, D, swa.SWA_F32, W, S, cross=True, ns=ns, R=R, sr0=sr0)
    for t in range(10):
        kf = t % 3 != 2
        q, k, v = frame_qkv(9, t, P, H, D, bf16=False)
        qd, kd, vd = (dev(x, torch.float32) for x in (q, k, v))
        out = torch.empty_like(qd)
        lse = torch.empty((H, P), dtype=torch.float32, device="cuda")
        gc.step(0, t, qd, kd, vd, kf, out, lse)
        ro, rl, pages = oc.step(t, q, k, v, kf)
        assert_close_f32(host(out), ro, f"out t={t}")
        assert_close_f32(host(lse), rl, f"lse t={t}")
        assert gc.pages() == oc.visible_pages()


def test_specials_across_tile_boundaries():
    # special rows 60..68 of a frame: in slot 0 they straddle the append's
    # work-group boundary at row 64 (each work-group retains the rows it is
    # about to overwrite), the 16-row V^T group boundary and the 64-key V^T
    # block boundary there; in slot 1 (rows 210..218) they lie inside one
    # work-group ([192, 224)) and inside the single V^T group [208, 224).
    # No scale frame, so both slots are reused.
    # Outputs, pages and the retained bytes against the oracle.
    P, H, D, W, S, ns, R, sr0 = 150, 2, 64, 2, 0, 9, 3, 60
    case(f"specials at rows {sr0}..{sr0 + ns - 1}, P={P} W={W} R={R}")
    gc, oc = _cache(P, H, D, swa.SWA_BF16, W, S, cross=True, ns=ns, R=R, sr0=sr0)
    frames = {}
    for t in range(12):
        kf = t % 3 != 2
        q, k, v = frame_qkv(8, t, P, H, D)
        frames[t] = (k, v)
        qd, kd, vd = dev(q), dev(k), dev(v)
        out = torch.empty_like(qd)
        lse = torch.empty((H, P), dtype=torch.float32, device="cuda")
        gc.step(0, t, qd, kd, vd, kf, out, lse)
        ro, rl, pages = oc.step(t, q, k, v, kf)
        assert_close_bf16(host(out), ro, f"out t={t}")
        assert np.abs(host(lse) - rl).max() <= lse_tol(sum(p[4] for p in pages))
        assert gc.pages() == oc.visible_pages()
    torch.cuda.synchronize()
    kr, vr = gc.region_views(0)
    K = kr.float().cpu().numpy()
    V = vt_keys(vr.float().cpu().numpy())
    base = gc.layout.special_row_base
    specials = [p for p in gc.pages() if p[1] != swa.SWA_REGION_FRAME]
    assert len(specials) == R
    for (f, _, _, row0, nrows) in specials:
        k, v = frames[f]
        assert np.array_equal(K[:, base + row0:base + row0 + nrows, :], k[sr0:sr0 + nrows].transpose(1, 0, 2))
        assert np.array_equal(V[:, :, base + row0:base + row0 + nrows], v[sr0:sr0 + nrows].transpose(1, 2, 0))


def test_frame_id_closed_form():
    # q = 0 makes every visible key weigh the same: the output is the mean
    # frame index of the visible rows, exact before the final bf16 rounding.
    P, H, D, W, S, ns, R = 29, 2, 64, 3, 2, 5, 3
    case("frame-id closed form")
    gc, oc = _cache(P, H, D, swa.SWA_BF16, W, S, cross=True, ns=ns, R=R)
    for t in range(14):
        kf = t % 3 != 2
        q = np.zeros((P, H, D), np.float32)
        k = frame_qkv(7, t, P, H, D)[1]
        v = np.full((P, H, D), float(t), np.float32)
        qd, kd, vd = dev(q), dev(k), dev(v)
        out = torch.empty_like(qd)
        gc.step(0, t, qd, kd, vd, kf, out, None)
        rows = [(f, nr) for (f, _, _, _, nr) in oc.step(t, q, k, v, kf)[2]]
        mean = sum(f * nr for f, nr in rows) / sum(nr for _, nr in rows)
        expect = bf16_round_f64(np.full((P, H, D), mean))
        assert np.array_equal(host(out), expect), (t, mean)


def test_nan_poisoned_pool():
    # Every byte of the pool starts as NaN: rows outside the visible segments
    # (page padding of the row space, unused slots, special ring) must never
    # reach the output.
    P, H, D, W, S = 50, 2, 64, 2, 1
    case("NaN-poisoned pool")
    gc, oc = _cache(P, H, D, swa.SWA_BF16, W, S, cross=True, ns=5, R=3)
    gc.pool.fill_(255)          # 0xFFFF is a bf16 NaN
    for t in range(10):
        kf = t % 4 != 3
        q, k, v = frame_qkv(8, t, P, H, D)
        qd, kd, vd = dev(q), dev(k), dev(v)
        out = torch.empty_like(qd)
        gc.step(0, t, qd, kd, vd, kf, out, None)
        ro, _, _ = oc.step(t, q, k, v, kf)
        assert_close_bf16(host(out), ro, f"t={t}")


def test_stream_equals_prefill_bf16():
    F, P, H, D, W, S = 8, 96, 2, 64, 3, 2
    case("stream == prefill bf16")
    q, k, v = chunk_qkv(9, F, P, H, D)
    pout = torch.empty((F * P, H, D), dtype=torch.bfloat16, device="cuda")
    swa.prefill_t(dev(q), dev(k), dev(v), F, P, W, 1, S, pout, None)
    gc, _ = _cache(P, H, D, swa.SWA_BF16, W, S)
    gc.set_splits(1)
    pg = host(pout)
    for t in range(F):
        rows = slice(t * P, (t + 1) * P)
        qd, kd, vd = dev(q[rows]), dev(k[rows]), dev(v[rows])
        out = torch.empty_like(qd)
        gc.step(0, t, qd, kd, vd, True, out, None)
        assert np.abs(host(out) - pg[rows]).max() <= 1e-2


def test_stream_equals_prefill_frame_blocks():
    # num_frame_per_block > 1 scales the window (2 blocks x 3 frames = 6
    # frames); the stream equals the masked prefill row block by row block.
    F, P, H, D, W, nfpb, S = 11, 70, 2, 64, 2, 3, 1
    case(f"stream==prefill bf16 F={F} P={P} W={W} nfpb={nfpb} S={S}")
    q, k, v = chunk_qkv(13, F, P, H, D)
    out_p = torch.empty((F * P, H, D), dtype=torch.bfloat16, device="cuda")
    swa.prefill_t(dev(q), dev(k), dev(v), F, P, W, nfpb, S, out_p, None)
    po, _ = prefill(q, k, v, F, P, W, nfpb, S)
    gc, oc = _cache(P, H, D, swa.SWA_BF16, W, S, nfpb=nfpb)
    for t in range(F):
        rows = slice(t * P, (t + 1) * P)
        qd, kd, vd = dev(q[rows]), dev(k[rows]), dev(v[rows])
        out = torch.empty_like(qd)
        gc.step(0, t, qd, kd, vd, True, out, None)
        ro, _, pages = oc.step(t, q[rows], k[rows], v[rows], True)
        assert gc.pages() == pages
        assert_close_bf16(host(out), ro, f"stream t={t}")
        assert_close_bf16(host(out), po[rows], f"stream==prefill t={t}")
        assert_close_bf16(host(out_p)[rows], po[rows], f"prefill t={t}")


def test_multi_layer_caches_are_independent():
    P, H, D = 33, 2, 64
    case("two layers")
    gc, _ = _cache(P, H, D, swa.SWA_BF16, 2, 1, num_layers=2)
    oc = [NaiveRingCache(CacheConfig(P=P, sliding_window_size=2, scale_frames=1)) for _ in range(2)]
    for t in range(6):
        for layer in range(2):
            q, k, v = frame_qkv(10 + layer, t, P, H, D)
            qd, kd, vd = dev(q), dev(k), dev(v)
            out = torch.empty_like(qd)
            gc.step(layer, t, qd, kd, vd, True, out, None)
            ro, _, _ = oc[layer].step(t, q, k, v, True)
            assert_close_bf16(host(out), ro, f"layer {layer} t={t}")


# ---------------------------------------------------------------------------
# 3-D RoPE
# ---------------------------------------------------------------------------

def _ulp_bf16(x):
    a = np.abs(x).astype(np.float32)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("t,bands", [(0, (12, 10, 10)), (5, (12, 10, 10)), (1999, (12, 10, 10)), (7, (0, 16, 16))])
def test_rope3d_apply(t, bands):
    # (0, 16, 16): 2-D RoPE (no temporal band)
    P, H, D = 1374, 4, 64
    case(f"rope3d t={t} bands={bands}")
    q, k, _ = frame_qkv(11, t, P, H, D)
    pos = frame_positions(t, 37, 37, 5)
    qd, kd = dev(q), dev(k)
    swa.rope3d_t(qd, kd, torch.from_numpy(pos).cuda(), bands)
    for got, x in ((host(qd), q), (host(kd), k)):
        ref = rope3d(x, pos, *bands)
        diff = np.abs(got - bf16_round_f64(ref))
        # one bf16 ulp of the exact value (floored at 2^-10 for values near 0,
        # where single-precision cancellation dominates)
        assert np.all(diff <= _ulp_bf16(np.maximum(np.abs(ref), 2.0 ** -10)) * 1.0001)


@pytest.mark.parametrize("bands", [(12, 10, 10), (0, 16, 16)])
def test_stream_with_rope_matches_oracle(bands):
    # (0, 16, 16): 2-D RoPE (height and width bands only) in the fused pass
    P, H, D, W, S = 1374, 2, 64, 4, 2
    case(f"stream + fused rope, bands {bands}")
    gc, oc = _cache(P, H, D, swa.SWA_BF16, W, S, rope=bands)
    for t in range(9):
        q, k, v = frame_qkv(12, t, P, H, D)
        pos = frame_positions(t, 37, 37, 5)
        qd, kd, vd = dev(q), dev(k), dev(v)
        out = torch.empty_like(qd)
        lse = torch.empty((H, P), dtype=torch.float32, device="cuda")
        gc.step(0, t, qd, kd, vd, True, out, lse, pos=torch.from_numpy(pos).cuda())
        # rotated exactly, then held in bf16 as the kernel holds them
        qr = bf16_round_f64(rope3d(q, pos, *bands))
        kr = bf16_round_f64(rope3d(k, pos, *bands))
        ro, rl, pages = oc.step(t, qr, kr, v, True)
        assert_close_bf16(host(out), ro, f"t={t}")
        assert np.abs(host(lse) - rl).max() <= lse_tol(sum(p[4] for p in pages))


# ---------------------------------------------------------------------------
# full-size workloads, sampled rows
# ---------------------------------------------------------------------------

SAMPLE_ROWS = np.array([0, 1, 4, 5, 63, 64, 127, 128, 700, 1279, 1280, 1300, 1343, 1344, 1373])


@pytest.mark.parametrize("H,splits", [(2, 0), (2, 3), (5, 0), (12, 0), (16, 0), (16, 1), (16, 7), (24, 0)])
def test_stream_work_split_sampled(H, splits):
    # The streaming decomposition: automatic columns over the (head, key
    # tile) space (heads cut mid-range, merged by a second kernel), and k
    # equal pieces per head.  The first steps have fewer tiles than columns.
    P, D, W, S = 1374, 64, 4, 2
    case(f"stream work split H={H} splits={splits}")
    gc, oc = _cache(P, H, D, swa.SWA_BF16, W, S)
    gc.set_splits(splits)
    for t in range(8):
        q, k, v = frame_qkv(20 + H, t, P, H, D)
        qd, kd, vd = dev(q), dev(k), dev(v)
        out = torch.full_like(qd, float("nan"))
        lse = torch.empty((H, P), dtype=torch.float32, device="cuda")
        gc.step(0, t, qd, kd, vd, True, out, lse)
        oc.append(t, k, v, True)
        oc.evict()
        ro, rl = oc.attend(q[SAMPLE_ROWS])
        assert_close_bf16(host(out)[SAMPLE_ROWS], ro, f"t={t}")
        assert np.abs(host(lse)[:, SAMPLE_ROWS] - rl).max() <= lse_tol(sum(p[4] for p in oc.visible_pages()))


def test_stream_step_full_size_sampled():
    # Single streaming step workload: P=1374, H=16, D=64, 8 scale + 16 window
    # frames (24 x 1374 = 32,976 visible keys), in the bench's launch config.
    P, H, D, W, S = 1374, 16, 64, 16, 8
    case("full-size stream step, sampled rows")
    gc, oc = _cache(P, H, D, swa.SWA_BF16, W, S)
    for t in range(30):
        q, k, v = frame_qkv(2, t % 97, P, H, D)
        qd, kd, vd = dev(q), dev(k), dev(v)
        out = torch.empty_like(qd)
        lse = torch.empty((H, P), dtype=torch.float32, device="cuda")
        gc.step(0, t, qd, kd, vd, True, out, lse)
        oc.append(t, k, v, True)
        oc.evict()
        if t in (0, 9, 29):
            assert sum(p[4] for p in oc.visible_pages()) == min(t + 1, 24) * P
            ro, rl = oc.attend(q[SAMPLE_ROWS])
            assert_close_bf16(host(out)[SAMPLE_ROWS], ro, f"t={t}")
            assert np.abs(host(lse)[:, SAMPLE_ROWS] - rl).max() <= lse_tol(min(t + 1, 24) * P)


def test_prefill_full_size_sampled():
    # Chunked prefill workload: 32 frames x 1374, window 8, 8 scale frames.
    F, P, H, D, W, S = 32, 1374, 16, 64, 8, 8
    case("full-size prefill, sampled rows")
    q, k, v = chunk_qkv(3, F, P, H, D)
    out = torch.empty((F * P, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, F * P), dtype=torch.float32, device="cuda")
    swa.prefill_t(dev(q), dev(k), dev(v), F, P, W, 1, S, out, lse)
    got, gl = host(out), host(lse)
    vis = frame_visibility(F, W, 1, S)
    fk = np.arange(F * P) // P
    for i in (0, 7, 8, 15, 16, 31):
        rows = i * P + SAMPLE_ROWS
        mask = np.broadcast_to(vis[i][fk][None, :], (len(rows), F * P))
        ro, rl = masked_attention(q[rows], k, v, mask)
        assert_close_bf16(got[rows], ro, f"frame {i}")
        assert np.abs(gl[:, rows] - rl).max() <= lse_tol(int(vis[i].sum()) * P), f"lse frame {i}"


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 32), ("bf16", 32)])
def test_prefill_large_chunk_layout(dtype, D):
    # 8 frames x 1024 tokens x 16 heads: large enough (at least 4096
    # work-groups of 32 rows) for the chunk layout to take 64-row append
    # blocks, in the dtypes and head sizes the full-size prefill does not
    # cover; sampled rows of three frames against the oracle.
    F, P, H, W, S = 8, 1024, 16, 2, 1
    case(f"prefill {dtype} D={D} F={F} P={P} H={H} (64-row layout blocks)")
    f32 = dtype == "f32"
    tdt = torch.float32 if f32 else torch.bfloat16
    q, k, v = chunk_qkv(11, F, P, H, D, bf16=not f32)
    out = torch.empty((F * P, H, D), dtype=tdt, device="cuda")
    lse = torch.empty((H, F * P), dtype=torch.float32, device="cuda")
    swa.prefill_t(dev(q, tdt), dev(k, tdt), dev(v, tdt), F, P, W, 1, S, out, lse)
    got, gl = host(out), host(lse)
    vis = frame_visibility(F, W, 1, S)
    fk = np.arange(F * P) // P
    sample = np.array([0, 1, 31, 32, 63, 64, 500, 1023])
    for i in (0, 3, 7):
        rows = i * P + sample
        mask = np.broadcast_to(vis[i][fk][None, :], (len(rows), F * P))
        ro, rl = masked_attention(q[rows], k, v, mask)
        if f32:
            assert_close_f32(got[rows], ro, f"frame {i}")
            assert_close_f32(gl[:, rows], rl, f"lse frame {i}")
        else:
            assert_close_bf16(got[rows], ro, f"frame {i}")
            assert np.abs(gl[:, rows] - rl).max() <= lse_tol(int(vis[i].sum()) * P), f"lse frame {i}"


# ---------------------------------------------------------------------------
# the offset softmax's recompute with a running max
# ---------------------------------------------------------------------------

def _spread_frames(t, P, H, D, gain, rng_id):
    """q along one direction u; frame t's keys along u with gain * t, so the
    scores of later frames exceed those of frame 0 by about
    1.44 * 12 * gain * t / 8 in log2 units (plus N(0,1) noise)."""
    rng = np.random.default_rng([rng_id, 99])
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q, k, v = frame_qkv(rng_id, t, P, H, D, bf16=False)
    q = 12.0 * u + 0.3 * q
    k = gain * t * u + 0.3 * k
    return tuple(bf16_round_f64(x).astype(np.float32) for x in (q, k, v))


@pytest.mark.parametrize("gain,splits,want_lse", [(4.0, 1, True), (4.0, 0, True), (4.0, 3, True), (2.0, 0, True),
                                                   (4.0, 0, False), (2.0, 0, False)])
def test_offset_softmax_spread_scores(gain, splits, want_lse):
    # gain 4: by frame 8 the window's scores exceed the first tile's maximum
    # by about 70 in log2 units, so the row sums pass 2^64 and the work items
    # are recomputed with the running-max softmax.  gain 2: about 35, so the
    # offset pass keeps probabilities up to 2^35 (no recompute).  Without an
    # LSE output the offset pass runs with Q pre-scaled.
    P, H, D, W, S = 150, 2, 64, 3, 1
    case(f"spread scores gain={gain} splits={splits} lse={want_lse}")
    gc, oc = _cache(P, H, D, swa.SWA_BF16, W, S)
    gc.set_splits(splits)
    for t in range(10):
        q, k, v = _spread_frames(t, P, H, D, gain, 51)
        qd, kd, vd = dev(q), dev(k), dev(v)
        out = torch.empty_like(qd)
        lse = torch.empty((H, P), dtype=torch.float32, device="cuda") if want_lse else None
        gc.step(0, t, qd, kd, vd, True, out, lse)
        ro, rl, pages = oc.step(t, q, k, v, True)
        assert_close_bf16(host(out), ro, f"out t={t}")
        if want_lse:
            # scores of this size (up to about 70 in log2 units): relative to |LSE|
            assert np.all(np.abs(host(lse) - rl) <= 2.0 ** -12 * np.abs(rl) + 1e-3), f"lse t={t}"


def test_offset_softmax_spread_scores_prefill():
    F, P, H, D, W, S = 9, 150, 2, 64, 3, 1
    case("spread scores, prefill")
    fr = [_spread_frames(t, P, H, D, 4.0, 52) for t in range(F)]
    q, k, v = (np.concatenate([f[i] for f in fr]) for i in range(3))
    ro, rl = prefill(q, k, v, F, P, W, 1, S)
    out = torch.empty((F * P, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, F * P), dtype=torch.float32, device="cuda")
    swa.prefill_t(dev(q), dev(k), dev(v), F, P, W, 1, S, out, lse)
    assert_close_bf16(host(out), ro, "out")
    assert np.all(np.abs(host(lse) - rl) <= 2.0 ** -12 * np.abs(rl) + 1e-3)
