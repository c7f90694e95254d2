"""Shared helpers of the GPU parity tests (imported by tests only)."""
import numpy as np
import torch

import sliding_window_kv_amd as swa

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5


def case(msg):
    print(f"[case] {msg}", flush=True)


def dev(x, dtype=torch.bfloat16):
    """numpy float32 (bf16-representable for bf16) -> device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(dtype)


def host(t):
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close_bf16(got, ref, what=""):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err.max() <= BF16_MAX_ABS, f"{what}: max abs {err.max():.3e}"
    assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean abs {err.mean():.3e}"
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
