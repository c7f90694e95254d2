"""GPU parity of token-level rolling-buffer decode with grouped-query heads
against the float64 oracle, through the C ABI (swa_decode_step)."""
import numpy as np
import pytest
import torch

import sliding_window_kv_amd as swa
from gpu_helpers import assert_close_bf16, case, dev, host, lse_tol, vt_keys
from oracle import RollingDecodeCache
from swa_synth import frame_qkv

pytestmark = pytest.mark.gpu


def _token(cfg, pos, B, Hq, Hkv, D):
    """q [B, Hq, D] and k, v [B, Hkv, D] of the token at position pos (bf16 values)."""
    _, k, v = frame_qkv(cfg, pos, B, Hkv, D)
    q = frame_qkv(cfg + 1000, pos, B, Hq, D)[0]
    return q, k, v


@pytest.mark.parametrize("B,Hq,Hkv,W,D", [(2, 8, 2, 37, 64), (3, 4, 4, 16, 64), (1, 32, 1, 50, 32), (2, 6, 3, 1, 64)])
def test_decode_matches_oracle(B, Hq, Hkv, W, D):
    # every position from 0 through two wraps of the buffer: warm-up
    # (pos < W), the first overwrite and the steady state
    case(f"decode B={B} Hq={Hq} Hkv={Hkv} W={W} D={D}")
    dc = swa.DecodeCache(B, Hq, Hkv, W, D)
    dc.cache.fill_(0xFF)                              # NaN bf16 everywhere: stale slots must never be read
    oc = [RollingDecodeCache(W, Hkv, D) for _ in range(B)]
    for pos in range(2 * W + 9):
        q, k, v = _token(40 + D, pos, B, Hq, Hkv, D)
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        dc.step(pos, dev(q), dev(k), dev(v), out, lse)
        ro = np.empty((B, Hq, D))
        rl = np.empty((B, Hq))
        for b in range(B):
            oc[b].append(pos, k[b], v[b])
            ro[b], rl[b] = oc[b].attend(pos, q[b])
        assert_close_bf16(host(out), ro, f"pos={pos}")
        assert np.abs(host(lse) - rl).max() <= lse_tol(min(pos + 1, W)), f"lse pos={pos}"
    # the buffers hold exactly the last W tokens' bf16 keys and values
    rows = (W + 64 + 63) // 64 * 64
    raw = dc.cache.view(torch.bfloat16).float().cpu().numpy()
    kb = raw[: B * Hkv * rows * D].reshape(B * Hkv, rows, D)
    vb = vt_keys(raw[dc.nbytes // 4:][: B * Hkv * D * rows].reshape(B * Hkv, rows // 64, D, 64))
    last = 2 * W + 8
    for p in range(max(0, last - W + 1), last + 1):
        _, k, v = _token(40 + D, p, B, Hq, Hkv, D)
        s = p % W
        assert np.array_equal(kb[:, s, :], k.reshape(B * Hkv, D))
        assert np.array_equal(vb[:, :, s], v.reshape(B * Hkv, D))


def test_decode_full_window_sampled():
    # W = 4096 slots, 32 query heads over 8 kv heads, past the first wrap
    B, Hq, Hkv, W, D = 1, 32, 8, 4096, 64
    case("decode W=4096 Hq=32 Hkv=8")
    dc = swa.DecodeCache(B, Hq, Hkv, W, D)
    oc = RollingDecodeCache(W, Hkv, D)
    check = {0, 1, 63, 64, 4095, 4096, 4097, 4200}
    for pos in range(4201):
        q, k, v = _token(48, pos % 997, B, Hq, Hkv, D)
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        dc.step(pos, dev(q), dev(k), dev(v), out, lse)
        oc.append(pos, k[0], v[0])
        if pos in check:
            ro, rl = oc.attend(pos, q[0])
            assert_close_bf16(host(out)[0], ro, f"pos={pos}")
            assert np.abs(host(lse)[0] - rl).max() <= lse_tol(min(pos + 1, W))


@pytest.mark.parametrize("B,Hq,Hkv,W,D", [(1, 3, 1, 12000, 32), (2, 6, 2, 9000, 64)])
def test_decode_long_window_many_pieces(B, Hq, Hkv, W, D):
    # more than 128 key tiles per buffer, so the merge folds its pieces in
    # more than one batch per lane; three query heads per kv head leave part
    # of the merge's last work-group without an item
    case(f"decode long window B={B} Hq={Hq} Hkv={Hkv} W={W} D={D}")
    dc = swa.DecodeCache(B, Hq, Hkv, W, D)
    oc = [RollingDecodeCache(W, Hkv, D) for _ in range(B)]
    check = {0, 130 * 64 - 1, W - 1, W, W + 77}
    toks = [_token(60 + D, i, B, Hq, Hkv, D) for i in range(389)]   # position p draws token p mod 389
    dtoks = [tuple(dev(x) for x in t) for t in toks]
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    for pos in range(W + 78):
        q, k, v = toks[pos % 389]
        dc.step(pos, *dtoks[pos % 389], out, lse)
        for b in range(B):
            oc[b].append(pos, k[b], v[b])
        if pos in check:
            for b in range(B):
                ro, rl = oc[b].attend(pos, q[b])
                assert_close_bf16(host(out)[b], ro, f"pos={pos} b={b}")
                assert np.abs(host(lse)[b] - rl).max() <= lse_tol(min(pos + 1, W)), f"lse pos={pos} b={b}"
