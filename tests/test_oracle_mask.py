"""Pins of the oracle's frame visibility and token mask (CPU only).

Each expected value here is built independently of the oracle's predicate:
from the guide's worked example typed out by hand, from banded/triangular
matrix constructions, or from a boolean reachability computation.
"""
import os

import numpy as np
import pytest

from oracle import frame_visibility, token_mask, window_frames

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([c == "1" for c in line])
    return np.array(rows, dtype=bool)


def _band(F, width):
    """ones where 0 <= i - j < width (np.tri differences)."""
    return (np.tri(F, F, 0, dtype=int) - np.tri(F, F, -width, dtype=int)).astype(bool)


def test_guide_example_frame_table():
    # Guide, "Manual Sliding-Window Mask Construction": 10 frames, window 4.
    gold = _golden_table("guide_example_frames.txt")
    assert gold.shape == (10, 10)
    assert np.array_equal(frame_visibility(10, 4, 1, 0), gold)
    assert np.array_equal(_band(10, 4), gold)


def test_guide_example_token_mask_full_size():
    # The same example at token level: [15600, 15600] booleans.
    F, fs = 10, 1560
    gold = _golden_table("guide_example_frames.txt")
    m = token_mask(F, fs, 4, 1, 0)
    assert m.shape == (F * fs, F * fs)
    blk = np.ones((fs, fs), dtype=bool)
    for i in range(F):
        row = m[i * fs:(i + 1) * fs]
        expect = np.concatenate([blk if gold[i, j] else ~blk for j in range(F)], axis=1)
        assert np.array_equal(row, expect), i
    # shape [1, 1, N, N] of the guide's builder is this mask with two unit dims
    assert m[None, None].shape == (1, 1, 15600, 15600)


@pytest.mark.parametrize("F,P", [(6, 21), (9, 4), (3, 1)])
def test_window_off_is_block_causal(F, P):
    # FAQ: sliding_window_size = -1 disables the window -> full causal.
    expect = np.kron(np.tril(np.ones((F, F), dtype=int)), np.ones((P, P), dtype=int)).astype(bool)
    assert np.array_equal(token_mask(F, P, -1, 1, 0), expect)
    # A window covering every frame gives the same mask.
    assert np.array_equal(token_mask(F, P, F, 1, 0), expect)
    assert np.array_equal(token_mask(F, P, F + 3, 1, 2), expect)


@pytest.mark.parametrize("W", [1, 2, 4, 7])
def test_token_level_swa(W):
    # P = 1, no scale frames: each token sees itself and the W-1 before it
    # (the explainer's definition of token-level sliding-window attention).
    N = 23
    m = token_mask(N, 1, W, 1, 0)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    assert np.array_equal(m, (j <= i) & (j >= i - W + 1))


def test_num_frame_per_block_scales_window():
    # window_start uses sliding_window_size * num_frame_per_block frames.
    assert np.array_equal(frame_visibility(12, 2, 3, 0), frame_visibility(12, 6, 1, 0))
    assert window_frames(6, 4) == 24
    assert window_frames(-1, 4) is None


def test_scale_frames_are_ored_in():
    F, W, S = 12, 3, 2
    vis = frame_visibility(F, W, 1, S)
    lower = np.tril(np.ones((F, F), dtype=bool))
    scale_cols = np.zeros((F, F), dtype=bool)
    scale_cols[:, :S] = True
    assert np.array_equal(vis, _band(F, W) | (lower & scale_cols))


def test_config3_visible_frame_pairs():
    # Chunked-prefill workload: 32 frames, window 8 blocks x 1, 8 scale frames.
    # Frames 0..15 see all earlier frames (i+1 each), frames 16..31 see 16.
    vis = frame_visibility(32, 8, 1, 8)
    assert vis.sum() == sum(i + 1 for i in range(16)) + 16 * 16 == 392
    assert np.tril(np.ones((32, 32))).sum() == 528


@pytest.mark.parametrize("bad", [0, -2, -5])
def test_invalid_window_rejected(bad):
    with pytest.raises(ValueError):
        frame_visibility(4, bad, 1, 0)


def test_receptive_field_grows_by_window_per_layer():
    # Explainer: stacking L layers of a width-W window reaches back L times the
    # window.  Exact boolean reachability of L mask hops from token i reaches
    # max(0, i - L*(W-1)), a span of L*(W-1)+1 <= L*W tokens.
    N, W = 64, 4                     # the explainer's toy window of 4
    m = token_mask(N, 1, W, 1, 0).astype(np.int64)
    reach = np.eye(N, dtype=np.int64)
    for L in range(1, 6):
        reach = ((reach @ m) > 0).astype(np.int64)
        for i in range(N):
            cols = np.nonzero(reach[i])[0]
            assert cols.min() == max(0, i - L * (W - 1))
            assert cols.max() == i
            assert len(cols) <= L * W
    # Mistral 7B figure in the explainer: 32 layers x 4096 = 131,072 tokens.
    assert 32 * 4096 == 131072
