"""Pins of the oracle's 3-D rotary embedding (CPU only)."""
import math
import os

import numpy as np

from oracle import rope3d

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _points():
    pts = []
    with open(os.path.join(GOLDEN, "rope3d_points.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                p, _, a = line.split()
                pts.append((int(p), float(a)))
    return pts


def test_hand_derived_angles():
    pos = np.array([[100, 50, 200]], dtype=np.int32)
    for p, angle in _points():
        x = np.zeros((1, 1, 64))
        x[0, 0, 2 * p] = 1.0                       # real part only
        y = rope3d(x, pos, 12, 10, 10)
        assert abs(y[0, 0, 2 * p] - math.cos(angle)) <= 1e-12
        assert abs(y[0, 0, 2 * p + 1] - math.sin(angle)) <= 1e-12
        x = np.zeros((1, 1, 64))
        x[0, 0, 2 * p + 1] = 1.0                   # imaginary part only
        y = rope3d(x, pos, 12, 10, 10)
        assert abs(y[0, 0, 2 * p] + math.sin(angle)) <= 1e-12
        assert abs(y[0, 0, 2 * p + 1] - math.cos(angle)) <= 1e-12
        # every other pair untouched (zero in, zero out)
        others = np.delete(y[0, 0], [2 * p, 2 * p + 1])
        assert np.all(others == 0.0)


def test_zero_position_is_identity():
    x = np.random.default_rng(0).standard_normal((7, 3, 64))
    assert np.array_equal(rope3d(x, np.zeros((7, 3), np.int32), 12, 10, 10), x)


def test_pair_norms_preserved():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 2, 64))
    pos = rng.integers(0, 2000, (9, 3)).astype(np.int32)
    y = rope3d(x, pos, 12, 10, 10)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.max(np.abs(nx - ny)) <= 1e-12


def test_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((5, 2, 64))
    k = rng.standard_normal((5, 2, 64))
    pq = rng.integers(0, 50, (5, 3)).astype(np.int32)
    pk = rng.integers(0, 50, (5, 3)).astype(np.int32)
    shift = np.array([[1900, 17, 29]], dtype=np.int32)
    s1 = np.einsum("nhd,nhd->nh", rope3d(q, pq, 12, 10, 10), rope3d(k, pk, 12, 10, 10))
    s2 = np.einsum("nhd,nhd->nh", rope3d(q, pq + shift, 12, 10, 10), rope3d(k, pk + shift, 12, 10, 10))
    assert np.max(np.abs(s1 - s2)) <= 1e-9


def test_temporal_only_reduces_to_1d_rope():
    # With every pair in the temporal band, the rotation is the 1-D rotary
    # embedding of RoFormer (Su et al.): pair i of a d-dim head turns by
    # m * base**(-2i/d), written here as explicit 2x2 rotation matrices.
    rng = np.random.default_rng(3)
    D = 64
    x = rng.standard_normal((4, 1, D))
    m = np.array([0, 1, 37, 1999])
    pos = np.stack([m, np.zeros(4, int), np.zeros(4, int)], 1).astype(np.int32)
    y = rope3d(x, pos, D // 2, 0, 0)
    for n in range(4):
        for i in range(D // 2):
            a = m[n] * 10000.0 ** (-2.0 * i / D)
            rot = np.array([[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]])
            expect = rot @ x[n, 0, 2 * i:2 * i + 2]
            assert np.max(np.abs(y[n, 0, 2 * i:2 * i + 2] - expect)) <= 1e-9
