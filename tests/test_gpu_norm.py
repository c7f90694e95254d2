"""GPU parity of the per-head q/k layer norm (standalone and fused into the
streaming step's append) against the float64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import sliding_window_kv_amd as swa
from gpu_helpers import assert_close_bf16, assert_close_f32, bf16_round_f64, case, dev, host, lse_tol
from oracle import CacheConfig, NaiveRingCache, head_layer_norm, rope3d
from swa_synth import frame_positions, frame_qkv, norm_weights

pytestmark = pytest.mark.gpu

EPS = 1e-5


def _ulp_bf16(a):
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _within_one_ulp(got, ref, what):
    # one bf16 ulp of the exact value, floored at 2^-10 near 0
    bound = _ulp_bf16(np.maximum(np.abs(ref), 2.0 ** -10)) * 1.0001
    diff = np.abs(got - ref)
    assert np.all(diff <= bound), f"{what}: worst {np.max(diff / bound):.3f} ulp"


@pytest.mark.parametrize("P,H,D", [(1374, 4, 64), (77, 3, 32)])
def test_qk_norm_apply_bf16(P, H, D):
    case(f"qk_norm bf16 P={P} H={H} D={D}")
    q, k, _ = frame_qkv(31, 0, P, H, D)
    q = q * 3.0 + 0.5                                  # rows with a mean and a scale to remove
    w = norm_weights(31, D)
    qd, kd = dev(q), dev(k)
    wd = torch.from_numpy(w).cuda()
    swa.qk_norm_t(qd, kd, wd, EPS)
    _within_one_ulp(host(qd), head_layer_norm(bf16_round_f64(q), w[0], w[1], EPS), "q")
    _within_one_ulp(host(kd), head_layer_norm(k, w[2], w[3], EPS), "k")


def test_qk_norm_apply_f32_and_single_tensor():
    P, H, D = 130, 2, 64
    case("qk_norm fp32, q only")
    q, k, _ = frame_qkv(32, 0, P, H, D, bf16=False)
    w = norm_weights(32, D)
    qd = dev(q, torch.float32)
    kd = dev(k, torch.float32)
    wd = torch.from_numpy(w).cuda()
    swa.qk_norm_t(qd, None, wd, EPS)
    assert_close_f32(host(qd), head_layer_norm(q, w[0], w[1], EPS), "q")
    assert np.array_equal(host(kd), k.astype(np.float64))          # untouched
    swa.qk_norm_t(None, kd, wd, EPS)
    assert_close_f32(host(kd), head_layer_norm(k, w[2], w[3], EPS), "k")


@pytest.mark.parametrize("rope", [(12, 10, 10), (0, 0, 0)])
def test_stream_normed_matches_oracle(rope):
    # The fused pre-attention pass: per-head norm of q and k, then 3-D RoPE
    # (when configured), then append, evict and attention, frame by frame.
    P, H, D, W, S = 1374, 2, 64, 4, 2
    case(f"stream with fused norm, rope={rope}")
    cfg = swa.make_config(P, H, D, sliding_window_size=W, scale_frames=S, rope=rope)
    gc = swa.SwaCache(cfg)
    oc = NaiveRingCache(CacheConfig(P=P, sliding_window_size=W, scale_frames=S))
    w = norm_weights(33, D)
    wd = torch.from_numpy(w).cuda()
    for t in range(8):
        q, k, v = frame_qkv(33, t, P, H, D)
        pos = frame_positions(t, 37, 37, 5)
        qd, kd, vd = dev(q), dev(k), dev(v)
        out = torch.empty_like(qd)
        lse = torch.empty((H, P), dtype=torch.float32, device="cuda")
        gc.step_normed(0, t, qd, kd, vd, wd, EPS, True, out, lse,
                       pos=torch.from_numpy(pos).cuda() if any(rope) else None)
        qn = head_layer_norm(q, w[0], w[1], EPS)
        kn = head_layer_norm(k, w[2], w[3], EPS)
        if any(rope):
            qn, kn = rope3d(qn, pos, *rope), rope3d(kn, pos, *rope)
        _within_one_ulp(host(qd), qn, f"q t={t}")
        # the cache holds bf16 keys: the oracle attends with k rounded the same way
        ro, rl, pages = oc.step(t, bf16_round_f64(qn), bf16_round_f64(kn), v, True)
        assert_close_bf16(host(out), ro, f"out t={t}")
        assert np.abs(host(lse) - rl).max() <= lse_tol(sum(p[4] for p in pages))


def test_fused_equals_separate_passes():
    # norm kernel + RoPE-fused append, against the single fused pass: the same
    # math with one more bf16 rounding in between, so outputs agree to bf16
    # tolerance and both match the oracle.
    P, H, D, W, S = 700, 2, 64, 3, 1
    rope = (12, 10, 10)
    case("fused vs separate pre-attention passes")
    cfg = swa.make_config(P, H, D, sliding_window_size=W, scale_frames=S, rope=rope)
    ga, gb = swa.SwaCache(cfg), swa.SwaCache(cfg)
    w = norm_weights(34, D)
    wd = torch.from_numpy(w).cuda()
    for t in range(5):
        q, k, v = frame_qkv(34, t, P, H, D)
        pos = torch.from_numpy(frame_positions(t, 26, 26, 24)).cuda()
        qa, ka, va = dev(q), dev(k), dev(v)
        qb, kb, vb = dev(q), dev(k), dev(v)
        oa, ob = torch.empty_like(qa), torch.empty_like(qb)
        ga.step_normed(0, t, qa, ka, va, wd, EPS, True, oa, None, pos=pos)
        swa.qk_norm_t(qb, kb, wd, EPS)
        gb.step(0, t, qb, kb, vb, True, ob, None, pos=pos)
        assert_close_bf16(host(oa), host(ob), f"t={t}")
        assert np.abs(host(qa) - host(qb)).max() <= 2 * _ulp_bf16(np.abs(host(qa)).max())
