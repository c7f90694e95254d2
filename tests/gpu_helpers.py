"""Shared helpers of the GPU parity tests (imported by tests only)."""
import os

import numpy as np
import torch

import sliding_window_kv_amd as swa

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5


def vt_keys(vb):
    """Transposed V read back from a cache region, in key order.

    vb: [N, rows / 64, D, 64], the documented storage of V^T (blocks of 64
    key positions, each [D][64]; key r at position r with bits 2 and 3
    swapped).  Returns [N, D, rows] with column r holding key r."""
    n, nb, d, _ = vb.shape
    by_pos = vb.transpose(0, 2, 1, 3).reshape(n, d, nb * 64)
    r = np.arange(nb * 64)
    return by_pos[:, :, (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1)]


def case(msg):
    print(f"[case] {msg}", flush=True)


def dev(x, dtype=torch.bfloat16):
    """numpy float32 (bf16-representable for bf16) -> device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dtype)


def host(t):
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy().astype(np.float64)


# Relative Frobenius error of a bf16 output: rounding the output to bf16
# and each probability before the PV product (both 2^-9 relative at most)
# give about 0.3%; the bound leaves three times that.  It is checked where
# the reference's RMS is at least 1e-3 (below that the absolute bounds
# above decide).
BF16_REL_FRO = 1e-2


def rel_fro(got, ref):
    """||got - ref|| / ||ref|| (Frobenius norms), or 0 for a zero reference."""
    n = float(np.linalg.norm(np.asarray(ref, np.float64)))
    return float(np.linalg.norm(np.asarray(got, np.float64) - ref)) / n if n > 0 else 0.0


def assert_close_bf16(got, ref, what=""):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err.max() <= BF16_MAX_ABS, f"{what}: max abs {err.max():.3e}"
    assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean abs {err.mean():.3e}"
    rel = rel_fro(got, ref)
    if os.environ.get("SWA_REPORT_REL"):
        print(f"[rel] {what}: {rel:.3e} (max abs {err.max():.3e})", flush=True)
    if np.sqrt(np.mean(np.square(ref))) >= 1e-3:
        assert rel <= BF16_REL_FRO, f"{what}: relative Frobenius error {rel:.3e}"
    return err.max(), err.mean()


def assert_close_f32(got, ref, what="", tol=F32_MAX_ABS):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err.max() <= tol, f"{what}: max abs {err.max():.3e}"
    return err.max()


def bf16_round_f64(x):
    """float64 -> nearest bfloat16 value (via torch's RNE conversion on CPU)."""
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.float32).to(torch.bfloat16).to(
        torch.float64).numpy()


def lse_tol(n_keys):
    """Tolerance on the fp32 LSE of one query row over n_keys visible keys.

    Per key, the kernel rounds each probability to bf16 (relative error up
    to 2^-9, independent across keys): about 1.1e-3 RMS, so the LSE moves by
    about 1.1e-3 * sqrt(sum_j a_j^2) with a_j the softmax weights.  For
    N(0,1) inputs (scaled scores ~ N(0, 1)) sum_j a_j^2 averages e / n over
    rows, with a wide spread when n is small (one key can dominate), so that
    term is bounded by 0.01 * sqrt(min(1, 8 / n)) (about six standard
    deviations).  Per query, the row sum is accumulated in fp32 over up to
    tens of thousands of terms and a rotated or normalised q is held in
    bf16; measured at full size these add up to about 2e-4, covered by a
    floor of 3e-4.  A lost or doubled 64-key tile moves the LSE by about
    64 / n (1.9e-3 at 32,976 keys), above the bound at every size; the q = 0
    closed-form tests check the key count exactly (LSE = ln n to 1e-5).
    """
    return 0.01 * float(np.sqrt(min(1.0, 8.0 / n_keys))) + 3e-4


def ulp_bf16(x):
    """Spacing of bfloat16 values at |x| (normal range)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)
