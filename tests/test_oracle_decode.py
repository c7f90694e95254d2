"""Pins of the oracle's token-level rolling-buffer decode (CPU only).

The explainer's rolling buffer writes position i to slot i mod W and never
holds more than W entries; a query sees itself and the W - 1 positions
before it; grouped-query heads share kv heads.  Pinned by the six-slot
widget, closed forms with q = 0 (uniform weights), the kv-group mapping,
and equality with the masked prefill at one token per frame (itself pinned
against the guide's mask example and torch SDPA).
"""
import math

import numpy as np
import pytest

from oracle import RollingDecodeCache, prefill


def test_six_slot_widget():
    c = RollingDecodeCache(W=6, Hkv=1, D=2)
    z = np.zeros((1, 2))
    for i in range(40):
        assert c.append(i, z, z) == i % 6
        live = [e for e in c.slots if e is not None]
        assert len(live) == min(i + 1, 6)                      # constant memory after warm-up
        assert sorted(e[0] for e in live) == list(range(max(0, i - 5), i + 1))


@pytest.mark.parametrize("W", [1, 4, 7])
def test_uniform_weights_give_the_window_mean(W):
    # q = 0: every visible key weighs the same, so with v = position the
    # output is the mean position of the window, (lo + pos) / 2, and the
    # log-sum-exp is log(count)
    D, Hq, Hkv = 8, 4, 2
    c = RollingDecodeCache(W=W, Hkv=Hkv, D=D)
    for pos in range(3 * W + 2):
        k = np.random.default_rng(pos).standard_normal((Hkv, D))
        c.append(pos, k, np.full((Hkv, D), float(pos)))
        out, lse = c.attend(pos, np.zeros((Hq, D)))
        lo = max(0, pos - W + 1)
        assert np.all(out == (lo + pos) / 2.0)
        assert np.abs(lse - math.log(pos - lo + 1)).max() <= 1e-12


def test_query_heads_read_their_kv_group():
    # kv head g holds v = g everywhere: with q = 0 query head h must return h // G
    Hq, Hkv, D, W = 8, 2, 4, 5
    c = RollingDecodeCache(W=W, Hkv=Hkv, D=D)
    for pos in range(7):
        v = np.repeat(np.arange(Hkv, dtype=np.float64)[:, None], D, axis=1)
        c.append(pos, np.ones((Hkv, D)), v)
    out, _ = c.attend(6, np.zeros((Hq, D)))
    assert np.array_equal(out[:, 0], np.arange(Hq) // (Hq // Hkv))


@pytest.mark.parametrize("W,Hq,Hkv", [(4, 2, 2), (3, 4, 2), (16, 8, 1)])
def test_equals_token_level_masked_prefill(W, Hq, Hkv):
    # one token per frame, no scale frames: the masked prefill's mask is the
    # token-level window (itself and W - 1 before); kv heads repeated per group
    N, D = 23, 16
    rng = np.random.default_rng(W * 100 + Hq)
    q = rng.standard_normal((N, Hq, D))
    k = rng.standard_normal((N, Hkv, D))
    v = rng.standard_normal((N, Hkv, D))
    G = Hq // Hkv
    po, pl = prefill(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), N, 1, W, 1, 0)
    c = RollingDecodeCache(W=W, Hkv=Hkv, D=D)
    for pos in range(N):
        c.append(pos, k[pos], v[pos])
        out, lse = c.attend(pos, q[pos])
        assert np.abs(out - po[pos]).max() <= 1e-12
        assert np.abs(lse - pl[:, pos]).max() <= 1e-12
