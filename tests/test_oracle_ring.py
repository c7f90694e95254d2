"""Pins of the oracle's naive ring cache (CPU only)."""
import numpy as np
import pytest

from oracle import REGION_FRAME, REGION_SPECIAL, CacheConfig, NaiveRingCache, RingError


def _kv(t, P=1, H=1, D=2):
    k = np.full((P, H, D), float(t))
    return k, -k


def test_six_slot_rolling_buffer_widget():
    # Explainer's widget: a six-slot buffer written at slot i modulo 6 that
    # never holds more than six entries.
    c = NaiveRingCache(CacheConfig(P=1, sliding_window_size=6, scale_frames=0))
    for t in range(40):
        c.append(t, *_kv(t), True)
        c.evict()
        pages = c.visible_pages()
        assert len(pages) == min(t + 1, 6)
        assert pages[-1] == (t, REGION_FRAME, t % 6, 0, 1)
        assert sorted(p[2] for p in pages) == sorted({f % 6 for f in range(max(0, t - 5), t + 1)})


def test_cache_size_is_constant_after_warmup():
    S, W = 3, 5
    c = NaiveRingCache(CacheConfig(P=2, sliding_window_size=W, scale_frames=S))
    for t in range(50):
        c.append(t, *_kv(t, P=2), True)
        c.evict()
        assert len(c.cached) == min(t + 1, S + W)
        slots = [p[2] for p in c.visible_pages()]
        assert len(set(slots)) == len(slots)
        assert max(slots) < S + W


def test_eviction_rule_literal():
    # Guide, "KV Cache Eviction Strategy": with more than window + scale frames
    # cached, positions [scale_frames, n_cached - window) are removed.
    c = NaiveRingCache(CacheConfig(P=1, sliding_window_size=3, scale_frames=2))
    evicted = []
    for t in range(6):
        c.append(t, *_kv(t), True)
        evicted.append(c.evict())
    assert evicted == [[], [], [], [], [], [2]]
    assert [e.frame for e in c.cached] == [0, 1, 3, 4, 5]
    c.append(6, *_kv(6), True)
    assert c.evict() == [3]
    assert [e.frame for e in c.cached] == [0, 1, 4, 5, 6]


def test_window_slots_follow_ordinal_modulo_window():
    S, W = 2, 4
    c = NaiveRingCache(CacheConfig(P=1, sliding_window_size=W, scale_frames=S))
    for t in range(20):
        c.append(t, *_kv(t), True)
        c.evict()
        assert c.cached[-1].slot == (t if t < S else S + (t - S) % W)


def test_non_keyframe_sees_cache_plus_itself_and_rolls_back():
    # Streaming branch of FlashInferBlock.forward: a non-keyframe is appended
    # with eviction deferred, attended, then rolled back.
    S, W = 1, 2
    c = NaiveRingCache(CacheConfig(P=1, sliding_window_size=W, scale_frames=S))
    for t in range(4):
        c.append(t, *_kv(t), True)
        c.evict()
    before = c.visible_pages()
    q = np.zeros((1, 1, 2))
    out, _, pages = c.step(4, q, *_kv(4), keyframe=False)
    assert [p[0] for p in pages] == [0, 2, 3, 4]
    assert pages[-1][2] == S + W                    # scratch slot
    # q = 0: uniform weights over the 4 visible frames' values
    assert np.allclose(out, -np.mean([0, 2, 3, 4]), atol=1e-12)
    assert c.visible_pages() == before
    with pytest.raises(RingError):
        c.rollback()


def test_cross_frame_special_fifo():
    P, ns, R = 6, 2, 3
    cfg = CacheConfig(P=P, sliding_window_size=2, scale_frames=1, cross_frame_special=True,
                      special_row0=0, special_rows=ns, max_special_frames=R)
    c = NaiveRingCache(cfg)
    for t in range(10):
        k = np.arange(P, dtype=float)[:, None, None] + 100 * t
        c.append(t, k, -k, True)
        c.evict()
    pages = c.visible_pages()
    # scale frame 0, the 3 most recently evicted frames (5,6,7), window 8,9
    assert [p[0] for p in pages] == [0, 5, 6, 7, 8, 9]
    sp = [p for p in pages if p[1] == REGION_SPECIAL]
    # evictions happen at t = 3..9 for frames 1..7 -> push indices 0..6
    assert [p[2] for p in sp] == [4 % R, 5 % R, 6 % R]
    assert [p[3] for p in sp] == [(4 % R) * ns, (5 % R) * ns, (6 % R) * ns]
    k, v = c.keys_values()
    # special rows are rows 0..ns-1 of the evicted frames
    assert list(k[P:P + ns, 0, 0]) == [500.0, 501.0]
    assert k.shape[0] == P + R * ns + 2 * P


def test_error_paths():
    c = NaiveRingCache(CacheConfig(P=1, sliding_window_size=-1, max_frames=3))
    with pytest.raises(RingError):
        c.rollback()
    for t in range(3):
        c.append(t, *_kv(t), True)
    with pytest.raises(RingError):
        c.append(3, *_kv(3), True)         # capacity with the window off
    c.append(5, *_kv(5), False)
    with pytest.raises(RingError):
        c.append(6, *_kv(6), False)        # second pending non-keyframe
    c.rollback()
    with pytest.raises(RingError):
        c.append(4, *_kv(4), False)        # frame index must increase


def test_reset_then_replay_reproduces_pages():
    cfg = CacheConfig(P=3, sliding_window_size=2, scale_frames=1, cross_frame_special=True,
                      special_rows=1, max_special_frames=2)
    c = NaiveRingCache(cfg)

    def run():
        seen = []
        for t in range(9):
            kf = t % 3 != 2
            c.append(t, *_kv(t, P=3), kf)
            if kf:
                c.evict()
            seen.append(c.visible_pages())
            if not kf:
                c.rollback()
        return seen

    a = run()
    c.reset()
    assert run() == a
