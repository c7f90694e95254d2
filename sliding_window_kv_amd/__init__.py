"""Python binding of libswa.so (gfx950 frame-block sliding-window attention).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Functions keep the C names of include/swa.h and take plain
integers (device addresses, sizes) and ctypes structures; ``SwaCache`` and
the ``*_t`` helpers accept torch tensors and pass their device addresses and
the current HIP stream.

The library must have been built (``python -m sliding_window_kv_amd.build``);
importing the binding without it raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libswa.so")
HEADER = os.path.join(ROOT, "include", "swa.h")

SWA_OK = 0
SWA_E_INVAL = -1
SWA_E_STATE = -2
SWA_E_CAPACITY = -3
SWA_E_UNSUPPORTED = -4
SWA_E_HIP = -5
SWA_BF16 = 0
SWA_F32 = 1
SWA_REGION_FRAME = 0
SWA_REGION_SPECIAL = 1


class swa_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_layers", "tokens_per_frame", "num_heads", "head_dim", "dtype", "sliding_window_size",
        "num_frame_per_block", "scale_frames", "cross_frame_special", "special_row0", "special_rows",
        "max_special_frames", "max_frames", "rope_pairs_t", "rope_pairs_h", "rope_pairs_w")] + [
        ("rope_theta", ctypes.c_float)]


class swa_page(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("frame", "region", "slot", "row0", "nrows")]


class swa_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "layer_bytes", "k_offset", "v_offset", "meta_offset", "work_offset", "work_bytes")] + [
        (n, ctypes.c_int32) for n in (
            "rows", "num_slots", "special_row_base", "elem_bytes", "window_frames", "scratch_slot")]


class SwaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_PROTOS = {
    "swa_cache_pool_bytes": (_sz, [ctypes.POINTER(swa_config)]),
    "swa_cache_create": (_i32, [ctypes.POINTER(swa_config), _vp, _sz, ctypes.POINTER(_vp)]),
    "swa_cache_destroy": (_i32, [_vp]),
    "swa_cache_layout": (_i32, [_vp, ctypes.POINTER(swa_layout)]),
    "swa_cache_set_splits": (_i32, [_vp, _i32]),
    "kvcache_reset": (_i32, [_vp, _vp]),
    "kvcache_append": (_i32, [_vp, _i32, _i64, _vp, _vp, _i32, _vp]),
    "kvcache_evict": (_i32, [_vp, _i32, _vp]),
    "kvcache_rollback": (_i32, [_vp, _i32, _vp]),
    "kvcache_attend": (_i32, [_vp, _i32, _vp, _vp, _vp, _vp]),
    "kvcache_visible_pages": (_i32, [_vp, _i32, ctypes.POINTER(swa_page), _i32, ctypes.POINTER(_i32)]),
    "kvcache_read_device_pages": (_i32, [_vp, _i32, ctypes.POINTER(swa_page), _i32, ctypes.POINTER(_i32), _vp]),
    "rope3d_apply": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _i32, _vp]),
    "swa_stream_step": (_i32, [_vp, _i32, _i64, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "swa_stream_step_normed": (_i32, [_vp, _i32, _i64, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _i32, _vp, _vp,
                                      _vp]),
    "qk_norm_apply": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, ctypes.c_float, _i32, _vp]),
    "swa_decode_cache_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "swa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "swa_decode_step": (_i32, [_vp, _sz, _i32, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                               _vp]),
    "swa_decode_step_noalloc": (_i32, [_vp, _sz, _i32, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "swa_prefill_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "swa_prefill_masked": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                  _vp, _sz, _vp]),
    "swa_prefill_mask": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    "swa_graph_create": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, ctypes.POINTER(_vp)]),
    "swa_graph_step": (_i32, [_vp, _i64, _i32, _vp]),
    "swa_graph_destroy": (_i32, [_vp]),
    "swa_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """The loaded libswa.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m sliding_window_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_functions():
    """Names of the functions declared in include/swa.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def check(rc):
    if rc != SWA_OK:
        raise SwaError(rc, lib().swa_last_error().decode())
    return rc


# ---- thin wrappers with the C names -------------------------------------------------

def swa_cache_pool_bytes(cfg):
    return lib().swa_cache_pool_bytes(ctypes.byref(cfg))


def swa_cache_create(cfg, dev_pool, pool_bytes):
    h = _vp()
    check(lib().swa_cache_create(ctypes.byref(cfg), dev_pool, pool_bytes, ctypes.byref(h)))
    return h


def swa_cache_destroy(h):
    return check(lib().swa_cache_destroy(h))


def swa_cache_layout(h):
    out = swa_layout()
    check(lib().swa_cache_layout(h, ctypes.byref(out)))
    return out


def swa_cache_set_splits(h, splits):
    return check(lib().swa_cache_set_splits(h, splits))


def kvcache_reset(h, stream=None):
    return check(lib().kvcache_reset(h, stream))


def kvcache_append(h, layer, frame_t, k, v, keyframe, stream=None):
    return check(lib().kvcache_append(h, layer, frame_t, k, v, int(keyframe), stream))


def kvcache_evict(h, layer, stream=None):
    return check(lib().kvcache_evict(h, layer, stream))


def kvcache_rollback(h, layer, stream=None):
    return check(lib().kvcache_rollback(h, layer, stream))


def kvcache_attend(h, layer, q, out, lse, stream=None):
    return check(lib().kvcache_attend(h, layer, q, out, lse, stream))


def kvcache_visible_pages(h, layer):
    n = _i32()
    check(lib().kvcache_visible_pages(h, layer, None, 0, ctypes.byref(n)))
    buf = (swa_page * max(1, n.value))()
    check(lib().kvcache_visible_pages(h, layer, buf, n.value, ctypes.byref(n)))
    return [(p.frame, p.region, p.slot, p.row0, p.nrows) for p in buf[:n.value]]


def kvcache_read_device_pages(h, layer, cap, stream=None):
    n = _i32()
    buf = (swa_page * max(1, cap))()
    check(lib().kvcache_read_device_pages(h, layer, buf, cap, ctypes.byref(n), stream))
    return [(p.frame, p.region, p.slot, p.row0, p.nrows) for p in buf[:min(cap, n.value)]], n.value


def rope3d_apply(q, k, pos, n_tokens, H, D, pt, ph, pw, theta, dtype, stream=None):
    return check(lib().rope3d_apply(q, k, pos, n_tokens, H, D, pt, ph, pw, theta, dtype, stream))


def swa_stream_step(h, layer, frame_t, q, k, v, pos, keyframe, out, lse, stream=None):
    return check(lib().swa_stream_step(h, layer, frame_t, q, k, v, pos, int(keyframe), out, lse, stream))


def swa_stream_step_normed(h, layer, frame_t, q, k, v, weights, eps, pos, keyframe, out, lse, stream=None):
    return check(lib().swa_stream_step_normed(h, layer, frame_t, q, k, v, weights, eps, pos, int(keyframe), out, lse,
                                              stream))


def qk_norm_apply(q, k, n_tokens, H, D, weights, eps, dtype, stream=None):
    return check(lib().qk_norm_apply(q, k, n_tokens, H, D, weights, eps, dtype, stream))


def swa_decode_cache_bytes(B, Hkv, W, D):
    return lib().swa_decode_cache_bytes(B, Hkv, W, D)


def swa_decode_workspace_bytes(Hq, Hkv, D):
    return lib().swa_decode_workspace_bytes(Hq, Hkv, D)


def swa_decode_step(cache, cache_bytes, B, Hq, Hkv, W, D, pos, q, k, v, out, lse, work, work_bytes, stream=None):
    return check(lib().swa_decode_step(cache, cache_bytes, B, Hq, Hkv, W, D, pos, q, k, v, out, lse, work, work_bytes,
                                       stream))


def swa_decode_step_noalloc(cache, cache_bytes, B, Hq, Hkv, W, D, pos, q, k, v, out, lse, stream=None):
    return check(lib().swa_decode_step_noalloc(cache, cache_bytes, B, Hq, Hkv, W, D, pos, q, k, v, out, lse, stream))


class DecodeCache:
    """Rolling buffers of B sequences for token decode (device memory from torch)."""

    def __init__(self, B, Hq, Hkv, W, D, device="cuda"):
        import torch
        self.B, self.Hq, self.Hkv, self.W, self.D = B, Hq, Hkv, W, D
        self.nbytes = swa_decode_cache_bytes(B, Hkv, W, D)
        self.wbytes = swa_decode_workspace_bytes(Hq, Hkv, D)
        if self.nbytes == 0 or self.wbytes == 0:
            raise SwaError(SWA_E_INVAL, "bad decode shape")
        self._buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        self._wbuf = torch.empty(self.wbytes + 256, dtype=torch.uint8, device=device)
        off = (-self._buf.data_ptr()) % 256
        self.cache = self._buf[off:off + self.nbytes]
        woff = (-self._wbuf.data_ptr()) % 256
        self.work = self._wbuf[woff:woff + self.wbytes]

    def step(self, pos, q, k, v, out, lse=None):
        swa_decode_step(_ptr(self.cache), self.nbytes, self.B, self.Hq, self.Hkv, self.W, self.D, pos, _ptr(q),
                        _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(self.work), self.wbytes, _stream())

    def step_noalloc(self, pos, q, k, v, out, lse=None):
        """The same step with the split partials in the library's static scratch (no workspace)."""
        swa_decode_step_noalloc(_ptr(self.cache), self.nbytes, self.B, self.Hq, self.Hkv, self.W, self.D, pos,
                                _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _stream())


def swa_prefill_workspace_bytes(F, P, H, D, dtype):
    return lib().swa_prefill_workspace_bytes(F, P, H, D, dtype)


def swa_prefill_masked(q, k, v, F, P, H, D, sws, nfpb, S, dtype, out, lse, ws, ws_bytes, stream=None):
    return check(lib().swa_prefill_masked(q, k, v, F, P, H, D, sws, nfpb, S, dtype, out, lse, ws, ws_bytes, stream))


def swa_prefill_mask(F, P, sws, nfpb, S, token_level, dev_out, stream=None):
    return check(lib().swa_prefill_mask(F, P, sws, nfpb, S, token_level, dev_out, stream))


def _ptr_array(ptrs):
    """A C array of device addresses (None entries become NULL), or None for None."""
    if ptrs is None:
        return None
    return (_vp * len(ptrs))(*[None if x is None else x for x in ptrs])


def swa_graph_create(h, q, k, v, out, lse, pos, norm_weights, eps):
    """q, k, v, out: lists of device addresses (one per layer); lse, norm_weights: such lists or None."""
    g = _vp()
    arrs = [_ptr_array(x) for x in (q, k, v, out, lse)]
    check(lib().swa_graph_create(h, *[ctypes.cast(a, _vp) if a is not None else None for a in arrs], pos,
                                 ctypes.cast(_ptr_array(norm_weights), _vp) if norm_weights is not None else None,
                                 eps, ctypes.byref(g)))
    return g


def swa_graph_step(g, frame_t, keyframe, stream=None):
    return check(lib().swa_graph_step(g, frame_t, int(keyframe), stream))


def swa_graph_destroy(g):
    return check(lib().swa_graph_destroy(g))


def swa_last_error():
    return lib().swa_last_error().decode()


# ---- torch conveniences (device memory and streams only) ------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_config(P, H, D, dtype=SWA_BF16, sliding_window_size=-1, num_frame_per_block=1, scale_frames=0,
                cross_frame_special=False, special_row0=0, special_rows=5, max_special_frames=1000,
                max_frames=64, num_layers=1, rope=(0, 0, 0), rope_theta=10000.0):
    c = swa_config()
    c.num_layers = num_layers
    c.tokens_per_frame = P
    c.num_heads = H
    c.head_dim = D
    c.dtype = dtype
    c.sliding_window_size = sliding_window_size
    c.num_frame_per_block = num_frame_per_block
    c.scale_frames = scale_frames
    c.cross_frame_special = int(bool(cross_frame_special))
    c.special_row0 = special_row0
    c.special_rows = special_rows
    c.max_special_frames = max_special_frames
    c.max_frames = max_frames
    c.rope_pairs_t, c.rope_pairs_h, c.rope_pairs_w = rope
    c.rope_theta = rope_theta
    return c


class SwaCache:
    """A cache whose device pool is a torch uint8 tensor on the current GPU."""

    def __init__(self, cfg, device="cuda"):
        import torch
        self.cfg = cfg
        nbytes = swa_cache_pool_bytes(cfg)
        if nbytes == 0:
            raise SwaError(SWA_E_INVAL, swa_last_error())
        self.pool = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        base = self.pool.data_ptr()
        off = (-base) % 256
        self.pool_view = self.pool[off:off + nbytes]
        self.handle = swa_cache_create(cfg, ctypes.c_void_p(self.pool_view.data_ptr()), nbytes)
        self.layout = swa_cache_layout(self.handle)

    def close(self):
        if self.handle is not None:
            swa_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def step(self, layer, t, q, k, v, keyframe=True, out=None, lse=None, pos=None):
        swa_stream_step(self.handle, layer, t, _ptr(q), _ptr(k), _ptr(v), _ptr(pos), keyframe, _ptr(out),
                        _ptr(lse), _stream())

    def step_normed(self, layer, t, q, k, v, weights, eps=1e-5, keyframe=True, out=None, lse=None, pos=None):
        """Streaming step with the per-head q/k layer norm fused into the append (weights: float [4, D])."""
        swa_stream_step_normed(self.handle, layer, t, _ptr(q), _ptr(k), _ptr(v), _ptr(weights), eps, _ptr(pos),
                               keyframe, _ptr(out), _ptr(lse), _stream())

    def append(self, layer, t, k, v, keyframe=True):
        kvcache_append(self.handle, layer, t, _ptr(k), _ptr(v), keyframe, _stream())

    def attend(self, layer, q, out, lse=None):
        kvcache_attend(self.handle, layer, _ptr(q), _ptr(out), _ptr(lse), _stream())

    def evict(self, layer):
        kvcache_evict(self.handle, layer, _stream())

    def rollback(self, layer):
        kvcache_rollback(self.handle, layer, _stream())

    def reset(self):
        kvcache_reset(self.handle, _stream())

    def set_splits(self, s):
        swa_cache_set_splits(self.handle, s)

    def pages(self, layer=0):
        return kvcache_visible_pages(self.handle, layer)

    def device_pages(self, layer=0, cap=4096):
        return kvcache_read_device_pages(self.handle, layer, cap, _stream())

    def region_views(self, layer=0):
        """(K [H, rows, D], V^T [H, rows / 64, D, 64]) tensors viewing the layer's rows.

        V^T is stored in blocks of 64 key positions (see swa_layout in swa.h)."""
        import torch
        L, c = self.layout, self.cfg
        dt = torch.bfloat16 if c.dtype == SWA_BF16 else torch.float32
        base = layer * L.layer_bytes
        H, D, rows = c.num_heads, c.head_dim, L.rows
        nb = H * rows * D * L.elem_bytes
        k = self.pool_view[base + L.k_offset: base + L.k_offset + nb].view(dt).view(H, rows, D)
        v = self.pool_view[base + L.v_offset: base + L.v_offset + nb].view(dt).view(H, rows // 64, D, 64)
        return k, v


class SwaGraph:
    """One captured streaming step of every layer of a SwaCache over fixed torch buffers.

    q, k, v, out: lists of num_layers tensors [P, H, D]; lse: list of float [H, P] tensors (or None
    entries) or None; pos: int32 [P, 3] tensor or None; norm_weights: list of float [4, D] tensors or
    None.  Write each frame's inputs into the buffers, then call step(t, keyframe).
    """

    def __init__(self, cache, q, k, v, out, lse=None, pos=None, norm_weights=None, eps=1e-5):
        self.cache = cache
        self._keep = (q, k, v, out, lse, pos, norm_weights)
        addr = lambda ts: None if ts is None else [None if t is None else t.data_ptr() for t in ts]
        self.handle = swa_graph_create(cache.handle, addr(q), addr(k), addr(v), addr(out), addr(lse), _ptr(pos),
                                       addr(norm_weights), eps)

    def step(self, t, keyframe=True):
        swa_graph_step(self.handle, t, keyframe, _stream())

    def close(self):
        if self.handle is not None:
            swa_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def prefill_t(q, k, v, F, P, sliding_window_size, num_frame_per_block, scale_frames, out, lse=None,
              workspace=None):
    """swa_prefill_masked over torch tensors [F*P, H, D] (workspace allocated if not given)."""
    import torch
    H, D = q.shape[1], q.shape[2]
    dtype = SWA_BF16 if q.dtype == torch.bfloat16 else SWA_F32
    need = swa_prefill_workspace_bytes(F, P, H, D, dtype)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    swa_prefill_masked(_ptr(q), _ptr(k), _ptr(v), F, P, H, D, sliding_window_size, num_frame_per_block,
                       scale_frames, dtype, _ptr(out), _ptr(lse), _ptr(workspace), need, _stream())
    return workspace


def rope3d_t(q, k, pos, pairs, theta=10000.0):
    import torch
    n, H, D = (q if q is not None else k).shape
    dtype = SWA_BF16 if (q if q is not None else k).dtype == torch.bfloat16 else SWA_F32
    rope3d_apply(_ptr(q), _ptr(k), _ptr(pos), n, H, D, pairs[0], pairs[1], pairs[2], theta, dtype, _stream())


def qk_norm_t(q, k, weights, eps=1e-5):
    """qk_norm_apply over torch tensors [n, H, D] in place (either may be None; weights float [4, D])."""
    import torch
    n, H, D = (q if q is not None else k).shape
    dtype = SWA_BF16 if (q if q is not None else k).dtype == torch.bfloat16 else SWA_F32
    qk_norm_apply(_ptr(q), _ptr(k), n, H, D, _ptr(weights), eps, dtype, _stream())


def prefill_mask_t(F, P, sliding_window_size, num_frame_per_block, scale_frames, token_level, out):
    swa_prefill_mask(F, P, sliding_window_size, num_frame_per_block, scale_frames, int(token_level), _ptr(out),
                     _stream())
