"""Pins of the oracle's per-head q/k layer norm (CPU only).

Each pin is a fact of the definition checked without re-using the oracle's
formula: a hand-derived example, the mean / mean-square identities of a
normalised row, shift and scale invariance, constant rows, the affine
weight/bias, and a cross-check against torch's float64 layer_norm.
"""
import math

import numpy as np
import pytest
import torch

from oracle import head_layer_norm


def _rng(seed):
    return np.random.default_rng(seed)


def test_hand_derived_example():
    # x = 1, 2, 3, 4: mean 2.5, biased variance 1.25, so (x - 2.5) / sqrt(1.25)
    # = (-3, -1, 1, 3) / sqrt(5) with no epsilon.
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    y = head_layer_norm(x, np.ones(4), np.zeros(4), eps=0.0)
    ref = np.array([-3.0, -1.0, 1.0, 3.0]) / math.sqrt(5.0)
    assert np.abs(y[0, 0] - ref).max() <= 1e-15


def test_row_moments_with_epsilon():
    # Unit weight, zero bias: every (token, head) row has mean 0 and mean
    # square var / (var + eps), computed from that row alone.
    x = _rng(1).standard_normal((7, 3, 64)) * _rng(2).uniform(0.1, 5.0, (7, 3, 1)) + 3.0
    eps = 1e-3
    y = head_layer_norm(x, np.ones(64), np.zeros(64), eps=eps)
    for n in range(7):
        for h in range(3):
            row = x[n, h]
            var = np.var(row)
            assert abs(y[n, h].mean()) <= 1e-12
            assert abs((y[n, h] ** 2).mean() - var / (var + eps)) <= 1e-12


def test_shift_and_scale_invariance():
    x = _rng(3).standard_normal((5, 2, 32))
    w, b = _rng(4).standard_normal(32), _rng(5).standard_normal(32)
    y = head_layer_norm(x, w, b, eps=0.0)
    assert np.abs(head_layer_norm(x + 7.25, w, b, eps=0.0) - y).max() <= 1e-12
    assert np.abs(head_layer_norm(3.5 * x, w, b, eps=0.0) - y).max() <= 1e-12
    # a negative scale flips the normalised row: -LN(x) before the affine part
    yn = head_layer_norm(-2.0 * x, np.ones(32), np.zeros(32), eps=0.0)
    assert np.abs(yn + head_layer_norm(x, np.ones(32), np.zeros(32), eps=0.0)).max() <= 1e-12


def test_constant_rows_give_the_bias():
    x = np.full((3, 4, 16), 2.75)
    b = _rng(6).standard_normal(16)
    y = head_layer_norm(x, _rng(7).standard_normal(16), b, eps=1e-5)
    assert np.array_equal(y, np.broadcast_to(b, y.shape))


def test_weight_scales_features_and_bias_shifts_them():
    x = _rng(8).standard_normal((4, 2, 64))
    w = np.arange(1, 65, dtype=np.float64) / 8.0
    b = -np.arange(64, dtype=np.float64) / 16.0
    plain = head_layer_norm(x, np.ones(64), np.zeros(64))
    y = head_layer_norm(x, w, b)
    assert np.abs(y - (plain * w[None, None, :] + b[None, None, :])).max() <= 1e-12


@pytest.mark.parametrize("D", [32, 64])
def test_matches_torch_layer_norm(D):
    x = _rng(9).standard_normal((11, 5, D))
    w, b = 1.0 + 0.1 * _rng(10).standard_normal(D), 0.1 * _rng(11).standard_normal(D)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (D,), torch.from_numpy(w), torch.from_numpy(b),
                                         eps=1e-5).numpy()
    assert np.abs(head_layer_norm(x, w, b, 1e-5) - ref).max() <= 1e-12
