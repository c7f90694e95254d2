"""Pins of the oracle's stream driver (stream_replay), CPU only.

stream_replay runs frames through one layer's naive ring cache the way the
streaming branch of FlashInferBlock.forward does (keyframe: append, evict,
attend; non-keyframe: append with eviction deferred, attend, roll back),
rotating k before it is cached and q before it attends.  It is pinned
against an independent path: the masked prefill over the rotated frames
(guide, "Mask Generation in CausalAttention"), whose row block t must equal
streaming step t; and against a hand-stepped cache with explicit rotations
for non-keyframes and retained special rows, where no prefill exists.
"""
import numpy as np
import pytest

from oracle import CacheConfig, NaiveRingCache, prefill, rope3d, stream_replay
from swa_synth import frame_positions, frame_qkv

F, GH, GW, NSP, H, D = 9, 3, 3, 3, 2, 16
P = NSP + GH * GW
BANDS = (3, 3, 2)


def _frames(cfg_id):
    data = [frame_qkv(cfg_id, t, P, H, D, bf16=False) for t in range(F)]
    pos = [frame_positions(t, GH, GW, NSP) for t in range(F)]
    return data, pos


@pytest.mark.parametrize("sws,nfpb,S", [(2, 2, 1), (1, 3, 0), (-1, 1, 0)])
def test_stream_replay_equals_prefill_with_rope(sws, nfpb, S):
    data, pos = _frames(41)
    cfg = CacheConfig(P=P, sliding_window_size=sws, num_frame_per_block=nfpb, scale_frames=S, max_frames=F)
    q = np.concatenate([d[0] for d in data])
    k = np.concatenate([d[1] for d in data])
    v = np.concatenate([d[2] for d in data])
    pa = np.concatenate(pos)
    po, pl = prefill(rope3d(q, pa, *BANDS), rope3d(k, pa, *BANDS), v, F, P, sws, nfpb, S)
    seen = 0
    for t, pages, out, lse in stream_replay(cfg, lambda t: data[t], F, pos_of=lambda t: pos[t], rope_pairs=BANDS):
        rows = slice(t * P, (t + 1) * P)
        assert np.abs(out - po[rows]).max() <= 1e-12
        assert np.abs(lse - pl[:, rows]).max() <= 1e-12
        seen += 1
    assert seen == F
    # the comparison has power: caching k unrotated changes step outputs by O(1)
    po_bad, _ = prefill(rope3d(q, pa, *BANDS), k, v, F, P, sws, nfpb, S)
    assert np.abs(po_bad - po).max() > 1e-2


def test_stream_replay_matches_hand_stepped_cache():
    # non-keyframes every third frame and retained special rows (no prefill
    # counterpart): each step equals NaiveRingCache.step on explicitly
    # rotated q and k
    data, pos = _frames(42)
    cfg = CacheConfig(P=P, sliding_window_size=2, scale_frames=1, cross_frame_special=True, special_row0=0,
                      special_rows=2, max_special_frames=3)
    key = lambda t: t % 3 != 2          # noqa: E731
    hand = NaiveRingCache(cfg)
    for t, pages, out, lse in stream_replay(cfg, lambda t: data[t], F, keyframe_of=key, pos_of=lambda t: pos[t],
                                            rope_pairs=BANDS):
        q, k, v = data[t]
        ho, hl, hp = hand.step(t, rope3d(q, pos[t], *BANDS), rope3d(k, pos[t], *BANDS), v, key(t))
        assert pages == hp
        assert np.abs(out - ho).max() <= 1e-12 and np.abs(lse - hl).max() <= 1e-12
    assert any(p[1] == 1 for p in pages)             # special entries were retained


def test_stream_replay_row_and_step_subsets():
    data, pos = _frames(43)
    cfg = CacheConfig(P=P, sliding_window_size=2, scale_frames=1, cross_frame_special=True, special_rows=2,
                      max_special_frames=2)
    key = lambda t: t % 4 != 3          # noqa: E731
    rows = np.array([0, 4, P - 1])
    full = list(stream_replay(cfg, lambda t: data[t], F, keyframe_of=key, pos_of=lambda t: pos[t],
                              rope_pairs=BANDS))
    part = list(stream_replay(cfg, lambda t: data[t], F, keyframe_of=key, pos_of=lambda t: pos[t],
                              rope_pairs=BANDS, record={2, 7}, rows=rows))
    for (t, pg, out, lse), (t2, pg2, out2, lse2) in zip(full, part):
        assert t == t2 and pg == pg2                  # unrecorded steps advance the ring identically
        if t in (2, 7):
            assert np.array_equal(out2, out[rows]) and np.array_equal(lse2, lse[:, rows])
        else:
            assert out2 is None and lse2 is None


def test_stream_replay_store_hook_rounds_rotated_q_and_k():
    # store models the precision of the tensors holding the rotated q and k
    data, pos = _frames(44)
    cfg = CacheConfig(P=P, sliding_window_size=2, scale_frames=1)
    halve = lambda x: np.round(x * 4.0) / 4.0           # noqa: E731  (a coarse grid, easy to check)
    hand = NaiveRingCache(cfg)
    for t, pages, out, lse in stream_replay(cfg, lambda t: data[t], F, pos_of=lambda t: pos[t], rope_pairs=BANDS,
                                            store=halve):
        q, k, v = data[t]
        ho, hl, _ = hand.step(t, halve(rope3d(q, pos[t], *BANDS)), halve(rope3d(k, pos[t], *BANDS)), v, True)
        assert np.abs(out - ho).max() <= 1e-12 and np.abs(lse - hl).max() <= 1e-12
