"""swa_decode_step_noalloc (split partials in the library's static scratch)
against swa_decode_step (caller workspace), through the C ABI, on a GPU.

Two runs in a row on the same process (the second with a smaller input),
each comparing the two entry points bit for bit at every position: same
kernels, same work split, so the same bits are expected."""
import numpy as np
import pytest
import torch

import sliding_window_kv_amd as swa
from gpu_helpers import case, dev, host
from swa_synth import frame_qkv

pytestmark = pytest.mark.gpu


def _run(B, Hq, Hkv, W, D, steps, cfg_id):
    case(f"decode noalloc vs workspace: B={B} Hq={Hq} Hkv={Hkv} W={W} D={D} steps={steps}")
    ref = swa.DecodeCache(B, Hq, Hkv, W, D)
    na = swa.DecodeCache(B, Hq, Hkv, W, D)          # its workspace is never passed
    ref.cache.zero_()                                 # rows never written compare equal too
    na.cache.zero_()
    for pos in range(steps):
        _, k, v = frame_qkv(cfg_id, pos, B, Hkv, D)
        q = frame_qkv(cfg_id + 1000, pos, B, Hq, D)[0]
        qd, kd, vd = dev(q), dev(k), dev(v)
        o1 = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
        o2 = torch.full_like(o1, float("nan"))
        l1 = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        l2 = torch.full_like(l1, float("nan"))
        ref.step(pos, qd, kd, vd, o1, l1)
        na.step_noalloc(pos, qd, kd, vd, o2, l2)
        assert torch.equal(o1, o2), f"out pos={pos}"
        assert torch.equal(l1, l2), f"lse pos={pos}"
        if pos % 7 == 0 or pos >= steps - 3:
            # the same position again without an LSE output (rewrites the same token)
            o3 = torch.full_like(o1, float("nan"))
            o4 = torch.full_like(o1, float("nan"))
            ref.step(pos, qd, kd, vd, o3, None)
            na.step_noalloc(pos, qd, kd, vd, o4, None)
            assert torch.equal(o3, o4) and torch.equal(o3, o1), f"out without lse pos={pos}"
    torch.cuda.synchronize()
    assert torch.equal(ref.cache, na.cache)           # the same rolling buffers (the new tokens' writes)


def test_noalloc_decode_matches_workspace_decode_twice():
    _run(4, 32, 8, 200, 64, 230, 61)                  # past a wrap of the 200-slot buffers
    _run(1, 8, 2, 70, 32, 80, 62)                     # second call sequence, smaller input


def test_noalloc_decode_split_columns():
    # enough sequences x kv heads x tiles for the automatic split to cut the
    # key range of every buffer into several pieces merged afterwards
    _run(16, 32, 8, 4096, 64, 4100, 63)
