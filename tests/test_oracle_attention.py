"""Pins of the oracle's masked attention (CPU only).

Checks against an independent library routine (torch's CPU float64
scaled_dot_product_attention), closed forms (uniform weights, log of the
visible-key count, a single visible key), invariants (rows sum to one,
key permutation), and stream == prefill in float64.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, strategies as st

from oracle import (CacheConfig, NaiveRingCache, frame_visibility, masked_attention, prefill,
                    token_mask)
from swa_synth import chunk_qkv, frame_qkv


def _sdpa(q, k, v, mask):
    tq = torch.from_numpy(np.asarray(q, np.float64)).permute(1, 0, 2)[None]
    tk = torch.from_numpy(np.asarray(k, np.float64)).permute(1, 0, 2)[None]
    tv = torch.from_numpy(np.asarray(v, np.float64)).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask))
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("F,P,H,D,W,nfpb,S", [
    (6, 21, 2, 32, 2, 1, 1),     # tiny fp32 workload shape
    (5, 7, 3, 16, -1, 1, 0),
    (7, 5, 2, 8, 1, 2, 2),
    (8, 3, 1, 64, 3, 1, 0),
])
def test_matches_torch_sdpa(F, P, H, D, W, nfpb, S):
    q, k, v = chunk_qkv(11, F, P, H, D, bf16=False)
    mask = token_mask(F, P, W, nfpb, S)
    out, _ = masked_attention(q, k, v, mask)
    ref = _sdpa(q, k, v, mask)
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_rows_sum_to_one_and_masked_weights_are_zero():
    F, P, H, D = 6, 21, 2, 32
    q, k, v = chunk_qkv(3, F, P, H, D, bf16=False)
    mask = token_mask(F, P, 2, 1, 1)
    _, _, a = masked_attention(q, k, v, mask, return_weights=True)
    assert np.max(np.abs(a.sum(axis=2) - 1.0)) <= 1e-12
    assert np.all(a[:, ~mask] == 0.0)


def test_constant_values_pass_through():
    F, P, H, D = 5, 6, 2, 8
    q, k, _ = chunk_qkv(4, F, P, H, D, bf16=False)
    v = np.ones_like(q)
    out, _ = masked_attention(q, k, v, token_mask(F, P, 2, 1, 1))
    assert np.max(np.abs(out - 1.0)) <= 1e-12


@pytest.mark.parametrize("W,S", [(2, 1), (3, 0), (-1, 0), (1, 2)])
def test_zero_query_closed_form(W, S):
    # q = 0 gives equal weights over the visible keys: the output is the mean
    # of the visible values and LSE = log(visible key count).  Values carry
    # their frame index, so a missing or extra frame is an O(1) error.
    F, P, H, D = 7, 4, 2, 8
    q = np.zeros((F * P, H, D))
    k = np.random.default_rng(0).standard_normal((F * P, H, D))
    v = np.repeat((np.arange(F * P) // P).astype(np.float64)[:, None, None], H, 1)
    v = np.repeat(v, D, 2)
    out, lse = masked_attention(q, k, v, token_mask(F, P, W, 1, S))
    for i in range(F):
        frames = [j for j in range(i + 1)
                  if W == -1 or j >= i - W + 1 or j < S]
        expect_mean = sum(frames) / len(frames)
        blk = out[i * P:(i + 1) * P]
        assert np.max(np.abs(blk - expect_mean)) <= 1e-12
        assert np.max(np.abs(lse[:, i * P:(i + 1) * P] - math.log(len(frames) * P))) <= 1e-12


def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 2, 4))
    k = rng.standard_normal((6, 2, 4))
    v = rng.standard_normal((6, 2, 4))
    mask = np.zeros((3, 6), dtype=bool)
    mask[0, 2] = mask[1, 5] = mask[2, 0] = True
    out, _ = masked_attention(q, k, v, mask)
    assert np.array_equal(out[0], v[2]) and np.array_equal(out[1], v[5]) and np.array_equal(out[2], v[0])


def test_key_permutation_invariance():
    F, P, H, D = 5, 6, 2, 16
    q, k, v = chunk_qkv(8, F, P, H, D, bf16=False)
    mask = token_mask(F, P, 2, 1, 1)
    perm = np.random.default_rng(1).permutation(F * P)
    o1, l1 = masked_attention(q, k, v, mask)
    o2, l2 = masked_attention(q, k[perm], v[perm], mask[:, perm])
    assert np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12


def test_brute_force_tiny():
    rng = np.random.default_rng(9)
    Nq, Nk, H, D = 3, 5, 2, 3
    q, k, v = (rng.standard_normal((n, H, D)) for n in (Nq, Nk, Nk))
    mask = rng.random((Nq, Nk)) < 0.6
    mask[:, 0] = True
    out, lse = masked_attention(q, k, v, mask)
    for h in range(H):
        for i in range(Nq):
            s = [sum(q[i, h, d] * k[j, h, d] for d in range(D)) / math.sqrt(D) if mask[i, j] else None
                 for j in range(Nk)]
            w = [math.exp(x) if x is not None else 0.0 for x in s]
            z = sum(w)
            for d in range(D):
                o = sum(w[j] * v[j, h, d] for j in range(Nk)) / z
                assert abs(o - out[i, h, d]) <= 1e-12
            assert abs(math.log(z) - lse[h, i]) <= 1e-12


def _stream_vs_prefill(F, P, H, D, W, nfpb, S, seed):
    q, k, v = chunk_qkv(seed, F, P, H, D, bf16=False)
    po, pl = prefill(q, k, v, F, P, W, nfpb, S)
    cache = NaiveRingCache(CacheConfig(P=P, sliding_window_size=W, num_frame_per_block=nfpb,
                                       scale_frames=S, max_frames=F + 1))
    for t in range(F):
        rows = slice(t * P, (t + 1) * P)
        o, l, pages = cache.step(t, q[rows], k[rows], v[rows], True)
        assert np.max(np.abs(o - po[rows])) <= 1e-12
        assert np.max(np.abs(l - pl[:, rows])) <= 1e-12
        vis = frame_visibility(F, W, nfpb, S)[t]
        assert [p[0] for p in pages] == list(np.nonzero(vis)[0])


def test_stream_equals_prefill_tiny_workload():
    # Tiny fp32 workload: 6 frames, P=21, H=2, D=32, window 2, 1 scale frame.
    _stream_vs_prefill(6, 21, 2, 32, 2, 1, 1, seed=1)


@given(F=st.integers(1, 9), P=st.integers(1, 6), H=st.integers(1, 2), D=st.sampled_from([2, 4, 8]),
       W=st.sampled_from([-1, 1, 2, 3, 5]), nfpb=st.integers(1, 2), S=st.integers(0, 3),
       seed=st.integers(0, 1000))
def test_stream_equals_prefill_property(F, P, H, D, W, nfpb, S, seed):
    _stream_vs_prefill(F, P, H, D, W, nfpb, S, seed)


def test_frame_qkv_is_seeded_and_bf16_exact():
    a = frame_qkv(2, 7, 5, 2, 8)
    b = frame_qkv(2, 7, 5, 2, 8)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
        # bf16-representable: low 16 bits of the float32 pattern are zero
        assert np.all((x.view(np.uint32) & 0xFFFF) == 0)
