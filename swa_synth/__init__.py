"""Seeded synthetic inputs shared by the oracle-side tests and the GPU-side tests.

This module only draws and encodes inputs. It holds none of the attention,
masking, cache or rotary arithmetic: both the float64 oracle and the HIP path
receive the arrays made here and nothing else from here.

Recipe (one generator per frame, so any frame can be re-drawn on its own):
  rng = numpy.random.default_rng([config_id, t])
  q, k, v = three successive standard_normal draws of shape [P, H, D], float32
  bf16 workloads round each value to bfloat16 (round to nearest, ties to even)
  and keep the rounded value, so both sides see bit-identical inputs.

Token rows of a frame: row 0 is the camera token, rows 1..n_reg the register
tokens, then the patch grid in row-major order.  3-D positions are (t, 0, 0)
for the special rows and (t, r, c) for the patch at grid row r, column c.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_bits",
    "bits_to_f32",
    "frame_qkv",
    "frame_positions",
    "chunk_qkv",
    "norm_weights",
]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32."""
    return bits_to_f32(bf16_bits(x))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values, round to nearest even.

    Adding 0x7FFF plus the kept part's lowest bit and dropping the low 16
    bits rounds to nearest, ties to even.  In 32-bit unsigned arithmetic this
    wraps only for NaN patterns, which are replaced by the quiet NaN after.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = u >> 16
    r &= 1
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    r = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """float32 values of bfloat16 bit patterns."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def frame_qkv(config_id: int, t: int, P: int, H: int, D: int, bf16: bool = True):
    """q, k, v of frame t as float32 arrays [P, H, D] (bf16-representable if bf16)."""
    rng = np.random.default_rng([int(config_id), int(t)])
    q = rng.standard_normal((P, H, D), dtype=np.float32)
    k = rng.standard_normal((P, H, D), dtype=np.float32)
    v = rng.standard_normal((P, H, D), dtype=np.float32)
    if bf16:
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    return q, k, v


def chunk_qkv(config_id: int, F: int, P: int, H: int, D: int, bf16: bool = True):
    """Frames 0..F-1 stacked into [F*P, H, D] float32 arrays."""
    qs, ks, vs = [], [], []
    for t in range(F):
        q, k, v = frame_qkv(config_id, t, P, H, D, bf16)
        qs.append(q)
        ks.append(k)
        vs.append(v)
    return np.concatenate(qs), np.concatenate(ks), np.concatenate(vs)


def frame_positions(t: int, grid_h: int, grid_w: int, n_special: int) -> np.ndarray:
    """int32 [P, 3] positions (t, r, c); special rows first at (t, 0, 0)."""
    P = n_special + grid_h * grid_w
    pos = np.zeros((P, 3), dtype=np.int32)
    pos[:, 0] = t
    j = np.arange(grid_h * grid_w)
    pos[n_special:, 1] = j // grid_w
    pos[n_special:, 2] = j % grid_w
    return pos


def norm_weights(config_id: int, D: int) -> np.ndarray:
    """float32 [4, D]: q weight, q bias, k weight, k bias (weights near 1, biases near 0)."""
    rng = np.random.default_rng([int(config_id), 7919])
    w = np.empty((4, D), dtype=np.float32)
    w[0] = 1.0 + 0.1 * rng.standard_normal(D, dtype=np.float32)
    w[1] = 0.1 * rng.standard_normal(D, dtype=np.float32)
    w[2] = 1.0 + 0.1 * rng.standard_normal(D, dtype=np.float32)
    w[3] = 0.1 * rng.standard_normal(D, dtype=np.float32)
    return w
