"""C-ABI checks that need no GPU: exported symbols, argument validation and
the host ring bookkeeping (page lists bit-exact against the oracle's naive
ring cache).  Caches are bookkeeping-only, or placed at a fake pool address
for argument checks that fail before anything is enqueued; no kernel runs."""
import ctypes

import numpy as np
import pytest
from hypothesis import given, strategies as st

import sliding_window_kv_amd as swa
from oracle import CacheConfig, NaiveRingCache, RingError


def test_library_exports_every_header_function():
    L = swa.lib()
    names = swa.header_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(L, n), n
        assert n in swa._PROTOS, n


def test_pool_bytes_and_layout():
    c = swa.make_config(1374, 16, 64, sliding_window_size=16, scale_frames=8)
    nb = swa.swa_cache_pool_bytes(c)
    h = swa.swa_cache_create(c, None, 0)
    L = swa.swa_cache_layout(h)
    assert L.num_slots == 8 + 16 + 1 and L.scratch_slot == 24
    assert L.window_frames == 16 and L.elem_bytes == 2
    assert L.rows % 64 == 0 and L.rows >= 25 * 1374 + 64
    assert L.v_offset == L.k_offset + 16 * L.rows * 64 * 2
    assert nb == L.work_offset + L.work_bytes
    swa.swa_cache_destroy(h)


@pytest.mark.parametrize("field,value,code", [
    ("sliding_window_size", 0, swa.SWA_E_INVAL),
    ("sliding_window_size", -3, swa.SWA_E_INVAL),
    ("head_dim", 48, swa.SWA_E_UNSUPPORTED),
    ("num_frame_per_block", 0, swa.SWA_E_INVAL),
    ("tokens_per_frame", 0, swa.SWA_E_INVAL),
    ("dtype", 7, swa.SWA_E_INVAL),
    ("scale_frames", -1, swa.SWA_E_INVAL),
])
def test_invalid_configs(field, value, code):
    c = swa.make_config(21, 2, 32, sliding_window_size=2, scale_frames=1)
    setattr(c, field, value)
    assert swa.swa_cache_pool_bytes(c) == 0
    with pytest.raises(swa.SwaError) as e:
        swa.swa_cache_create(c, None, 0)
    assert e.value.code == code
    assert swa.swa_last_error() != ""


def test_special_rows_must_fit_and_rope_bands_must_sum():
    c = swa.make_config(4, 2, 32, sliding_window_size=2, cross_frame_special=True, special_rows=5)
    with pytest.raises(swa.SwaError):
        swa.swa_cache_create(c, None, 0)
    c = swa.make_config(21, 2, 32, sliding_window_size=2, rope=(5, 5, 5))
    with pytest.raises(swa.SwaError):
        swa.swa_cache_create(c, None, 0)


def test_bookkeeping_cache_refuses_device_work():
    c = swa.make_config(21, 2, 32, sliding_window_size=2, scale_frames=1)
    h = swa.swa_cache_create(c, None, 0)
    with pytest.raises(swa.SwaError) as e:
        swa.swa_stream_step(h, 0, 0, ctypes.c_void_p(8), ctypes.c_void_p(8), ctypes.c_void_p(8), None, 1,
                            ctypes.c_void_p(8), None)
    assert e.value.code == swa.SWA_E_STATE
    with pytest.raises(swa.SwaError) as e:
        swa.kvcache_read_device_pages(h, 0, 16)
    assert e.value.code == swa.SWA_E_STATE
    with pytest.raises(swa.SwaError) as e:
        swa.kvcache_append(h, 5, 0, None, None, True)        # layer out of range
    assert e.value.code == swa.SWA_E_INVAL


def test_attend_refused_while_an_eviction_is_pending():
    # window 2, 1 scale frame: the 4th keyframe fills the window past 2
    # frames; until kvcache_evict runs, attending (and reading the device
    # page list) is refused, as the oracle refuses it
    ora, h = _pair(5, 2, 1, True, 2, 3)
    p = ctypes.c_void_p(256)
    try:
        for t in range(3):
            ora.append(t, *_kv(5), True)
            ora.evict()
            swa.kvcache_append(h, 0, t, None, None, True)
            swa.kvcache_evict(h, 0)
        ora.append(3, *_kv(5), True)
        swa.kvcache_append(h, 0, 3, None, None, True)
        with pytest.raises(RingError):
            ora.attend(np.zeros((5, 1, 1)))
        for call in (lambda: swa.kvcache_attend(h, 0, p, p, None),
                     lambda: swa.kvcache_read_device_pages(h, 0, 16)):
            with pytest.raises(swa.SwaError) as e:
                call()
            assert e.value.code == swa.SWA_E_STATE and "eviction is pending" in str(e.value)
        ora.evict()
        swa.kvcache_evict(h, 0)
        ora.attend(np.zeros((5, 1, 1)))
        with pytest.raises(swa.SwaError) as e:          # now only the missing pool stops it
            swa.kvcache_attend(h, 0, p, p, None)
        assert e.value.code == swa.SWA_E_STATE and "bookkeeping-only" in str(e.value)
        assert swa.kvcache_visible_pages(h, 0) == ora.visible_pages()
    finally:
        swa.swa_cache_destroy(h)


def test_row_space_limit():
    # one head's K / V^T region is addressed with 32-bit offsets: rows x D x
    # element bytes must stay below 2 GiB (window off, 30,000 frames of 1374
    # tokens at D = 64 would be 5.3 GB per head)
    big = swa.make_config(1374, 1, 64, sliding_window_size=-1, max_frames=30000)
    assert swa.swa_cache_pool_bytes(big) == 0
    with pytest.raises(swa.SwaError) as e:
        swa.swa_cache_create(big, None, 0)
    assert e.value.code == swa.SWA_E_INVAL
    ok = swa.make_config(1374, 1, 64, sliding_window_size=-1, max_frames=12000)   # 2.1e9 B: just under
    assert swa.swa_cache_pool_bytes(ok) > 0
    f32 = swa.make_config(1374, 1, 64, dtype=swa.SWA_F32, sliding_window_size=-1, max_frames=12000)
    assert swa.swa_cache_pool_bytes(f32) == 0
    rows_max = (1 << 31) // (64 * 2)                  # bf16, D = 64
    assert swa.swa_prefill_workspace_bytes(1, rows_max - 200, 1, 64, swa.SWA_BF16) > 0
    assert swa.swa_prefill_workspace_bytes(1, rows_max, 1, 64, swa.SWA_BF16) == 0
    assert swa.swa_decode_cache_bytes(1, 1, rows_max - 200, 64) > 0
    assert swa.swa_decode_cache_bytes(1, 1, rows_max, 64) == 0


def test_prefill_argument_checks():
    need = swa.swa_prefill_workspace_bytes(4, 10, 2, 64, swa.SWA_BF16)
    assert need > 0 and need % 256 == 0
    assert swa.swa_prefill_workspace_bytes(4, 10, 2, 48, swa.SWA_BF16) == 0
    p = ctypes.c_void_p(256)
    with pytest.raises(swa.SwaError) as e:
        swa.swa_prefill_masked(p, p, p, 4, 10, 2, 64, 0, 1, 0, swa.SWA_BF16, p, None, p, need)
    assert e.value.code == swa.SWA_E_INVAL
    with pytest.raises(swa.SwaError) as e:
        swa.swa_prefill_masked(p, p, p, 4, 10, 2, 64, 2, 1, 0, swa.SWA_BF16, p, None, p, need - 1)
    assert e.value.code == swa.SWA_E_INVAL
    with pytest.raises(swa.SwaError) as e:
        swa.rope3d_apply(p, p, p, 10, 2, 64, 10, 10, 10, 1e4, swa.SWA_BF16)
    assert e.value.code == swa.SWA_E_INVAL


def test_qk_norm_argument_checks():
    p = ctypes.c_void_p(256)
    for args, code in [((p, p, 10, 2, 64, None, 1e-5, swa.SWA_BF16), swa.SWA_E_INVAL),   # no weights
                       ((None, None, 10, 2, 64, p, 1e-5, swa.SWA_BF16), swa.SWA_E_INVAL),  # no tensors
                       ((p, p, 10, 2, 64, p, -1.0, swa.SWA_BF16), swa.SWA_E_INVAL),        # eps < 0
                       ((p, p, -1, 2, 64, p, 1e-5, swa.SWA_BF16), swa.SWA_E_INVAL),        # bad shape
                       ((p, p, 10, 2, 48, p, 1e-5, swa.SWA_BF16), swa.SWA_E_UNSUPPORTED),  # head_dim 48
                       ((p, p, 10, 2, 64, p, 1e-5, 7), swa.SWA_E_INVAL)]:                  # bad dtype
        with pytest.raises(swa.SwaError) as e:
            swa.qk_norm_apply(*args)
        assert e.value.code == code
    swa.qk_norm_apply(p, p, 0, 2, 64, p, 1e-5, swa.SWA_BF16)                               # nothing to do
    # the fused step validates its norm arguments before touching the cache
    c = swa.make_config(10, 2, 64, sliding_window_size=2, scale_frames=1)
    h = swa.swa_cache_create(c, None, 0)
    try:
        with pytest.raises(swa.SwaError) as e:
            swa.swa_stream_step_normed(h, 0, 0, p, p, p, None, 1e-5, None, True, p, None)
        assert e.value.code == swa.SWA_E_INVAL
        with pytest.raises(swa.SwaError) as e:
            swa.swa_stream_step_normed(h, 0, 0, p, p, p, p, -1.0, None, True, p, None)
        assert e.value.code == swa.SWA_E_INVAL
        with pytest.raises(swa.SwaError) as e:                                              # bookkeeping-only cache
            swa.swa_stream_step_normed(h, 0, 0, p, p, p, p, 1e-5, None, True, p, None)
        assert e.value.code == swa.SWA_E_STATE
    finally:
        swa.swa_cache_destroy(h)


def test_decode_argument_checks():
    p = ctypes.c_void_p(256)
    assert swa.swa_decode_cache_bytes(1, 8, 4096, 48) == 0
    assert swa.swa_decode_workspace_bytes(33, 1, 64) == 0          # more than 32 query heads per kv head
    assert swa.swa_decode_workspace_bytes(6, 4, 64) == 0           # not a multiple
    need = swa.swa_decode_cache_bytes(1, 1, 16, 64)
    # K and V^T of 1 x 1 heads, 16 slots rounded up plus 64 rows of padding, 64 bf16 each
    assert need == 2 * ((128 * 64 * 2 + 255) // 256 * 256)
    work = swa.swa_decode_workspace_bytes(1, 1, 64)
    for args, code in [((None, need, 1, 1, 1, 16, 64, 0), swa.SWA_E_INVAL),          # no cache
                       ((p, need - 1, 1, 1, 1, 16, 64, 0), swa.SWA_E_INVAL),         # cache too small
                       ((p, need, 1, 1, 1, 16, 64, -1), swa.SWA_E_INVAL),            # negative position
                       ((p, need, 1, 3, 2, 16, 64, 0), swa.SWA_E_INVAL),             # Hq not a multiple of Hkv
                       ((p, need, 1, 1, 1, 0, 64, 0), swa.SWA_E_INVAL),              # empty window
                       ((p, need, 1, 1, 1, 16, 48, 0), swa.SWA_E_UNSUPPORTED)]:      # head_dim 48
        with pytest.raises(swa.SwaError) as e:
            swa.swa_decode_step(*args, p, p, p, p, None, p, work)
        assert e.value.code == code
    with pytest.raises(swa.SwaError) as e:                                            # workspace too small
        swa.swa_decode_step(p, need, 1, 1, 1, 16, 64, 0, p, p, p, p, None, p, work - 1)
    assert e.value.code == swa.SWA_E_INVAL


def test_decode_noalloc_argument_checks():
    # the allocation-free decode rejects argument errors and group sizes whose
    # split partials exceed its 16 MiB static scratch before touching the GPU
    p = ctypes.c_void_p(256)
    need = swa.swa_decode_cache_bytes(1, 4, 64, 64)
    for args, code in [((p, need, 1, 64, 4, 64, 64, 0), swa.SWA_E_CAPACITY),     # 16 query heads per kv head, D 64
                       ((p, need, 1, 62, 2, 64, 32, 0), swa.SWA_E_CAPACITY),     # 31 per kv head, D 32
                       ((p, need, 1, 6, 4, 64, 64, 0), swa.SWA_E_INVAL),         # Hq not a multiple of Hkv
                       ((p, need, 1, 8, 4, 64, 48, 0), swa.SWA_E_UNSUPPORTED)]:  # head_dim 48
        with pytest.raises(swa.SwaError) as e:
            swa.swa_decode_step_noalloc(*args, p, p, p, p, None)
        assert e.value.code == code


def _pair(P, W, S, cross, ns, R, max_frames=50):
    ocfg = CacheConfig(P=P, sliding_window_size=W, scale_frames=S, cross_frame_special=cross,
                       special_row0=0, special_rows=ns, max_special_frames=R, max_frames=max_frames)
    c = swa.make_config(P, 1, 32, sliding_window_size=W, scale_frames=S, cross_frame_special=cross,
                        special_rows=ns, max_special_frames=R, max_frames=max_frames)
    return NaiveRingCache(ocfg), swa.swa_cache_create(c, None, 0)


def _kv(P):
    z = np.zeros((P, 1, 1))
    return z, z


OPS = st.lists(st.sampled_from(["key", "key", "key", "nonkey", "evict", "rollback", "reset", "stale"]),
               min_size=1, max_size=60)


@given(P=st.integers(5, 9), W=st.sampled_from([-1, 1, 2, 3, 5]), S=st.integers(0, 3),
       cross=st.booleans(), ns=st.integers(1, 3), R=st.integers(1, 4), ops=OPS)
def test_page_lists_bit_exact_vs_oracle(P, W, S, cross, ns, R, ops):
    ora, h = _pair(P, W, S, cross, ns, R, max_frames=12)
    t = 0
    try:
        for op in ops:
            expect_err = None
            try:
                if op == "key":
                    ora.append(t, *_kv(P), True)
                elif op == "nonkey":
                    ora.append(t, *_kv(P), False)
                elif op == "stale":
                    ora.append(t - 2, *_kv(P), True)
                elif op == "evict":
                    ora.evict()
                elif op == "rollback":
                    ora.rollback()
                else:
                    ora.reset()
            except RingError:
                expect_err = True
            got_err = None
            try:
                if op in ("key", "nonkey", "stale"):
                    swa.kvcache_append(h, 0, t if op != "stale" else t - 2, None, None, op != "nonkey")
                elif op == "evict":
                    swa.kvcache_evict(h, 0)
                elif op == "rollback":
                    swa.kvcache_rollback(h, 0)
                else:
                    swa.kvcache_reset(h)
            except swa.SwaError:
                got_err = True
            assert got_err == expect_err, op
            if op in ("key", "nonkey"):
                t += 1
            if op == "reset":
                t = 0
            assert swa.kvcache_visible_pages(h, 0) == ora.visible_pages()
    finally:
        swa.swa_cache_destroy(h)


def test_long_stream_with_specials_bit_exact():
    # Ragged cross-frame-special workload shape: window 16, 8 scale frames,
    # 5 special rows, every third frame a non-keyframe; R reduced to 40 so
    # the special ring wraps several times within 400 frames.
    ora, h = _pair(1405, 16, 8, True, 5, 40)
    try:
        for t in range(400):
            kf = t % 3 != 2
            ora.append(t, *_kv(1405), kf)
            swa.kvcache_append(h, 0, t, None, None, kf)
            if kf:
                ora.evict()
                swa.kvcache_evict(h, 0)
            assert swa.kvcache_visible_pages(h, 0) == ora.visible_pages()
            if not kf:
                ora.rollback()
                swa.kvcache_rollback(h, 0)
    finally:
        swa.swa_cache_destroy(h)


def test_capacity_error_with_window_off():
    ora, h = _pair(5, -1, 0, False, 1, 1, max_frames=3)
    for t in range(3):
        swa.kvcache_append(h, 0, t, None, None, True)
    with pytest.raises(swa.SwaError) as e:
        swa.kvcache_append(h, 0, 3, None, None, True)
    assert e.value.code == swa.SWA_E_CAPACITY
    # a non-keyframe still fits in the scratch slot
    swa.kvcache_append(h, 0, 4, None, None, False)
    assert swa.kvcache_visible_pages(h, 0)[-1] == (4, 0, 3, 0, 5)
    swa.swa_cache_destroy(h)


def test_graph_argument_checks():
    # a cache over a fake (never dereferenced) pool address: every call below
    # fails its argument or state check before anything is enqueued
    fake = ctypes.c_void_p(1 << 20)
    a4 = [256, 256]
    c = swa.make_config(21, 2, 32, num_layers=2, sliding_window_size=2, scale_frames=1, dtype=swa.SWA_F32)
    h = swa.swa_cache_create(c, fake, swa.swa_cache_pool_bytes(c))
    with pytest.raises(swa.SwaError) as e:
        swa.swa_graph_create(h, a4, a4, a4, a4, None, None, None, 1e-5)
    assert e.value.code == swa.SWA_E_UNSUPPORTED
    swa.swa_cache_destroy(h)
    c = swa.make_config(21, 2, 32, num_layers=2, sliding_window_size=2, scale_frames=1)
    h = swa.swa_cache_create(c, fake, swa.swa_cache_pool_bytes(c))
    for args in [([256, None], a4, a4, a4, None, None, None, 1e-5),          # null tensor
                 (a4, a4, a4, a4, None, ctypes.c_void_p(256), None, 1e-5),  # positions without rope bands
                 (a4, a4, a4, a4, None, None, a4, -1.0),                    # negative epsilon
                 (a4, a4, a4, a4, None, None, [256, None], 1e-5)]:          # null norm weights
        with pytest.raises(swa.SwaError) as e:
            swa.swa_graph_create(h, *args)
        assert e.value.code == swa.SWA_E_INVAL
    swa.swa_cache_destroy(h)
    d = swa.swa_cache_create(c, None, 0)
    with pytest.raises(swa.SwaError) as e:
        swa.swa_graph_create(d, a4, a4, a4, a4, None, None, None, 1e-5)
    assert e.value.code == swa.SWA_E_STATE
    with pytest.raises(swa.SwaError) as e:
        swa.swa_graph_step(None, 0, 1)
    assert e.value.code == swa.SWA_E_INVAL
    swa.swa_cache_destroy(d)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    # no fallback of any kind: without the built library every entry point
    # refuses to run
    monkeypatch.setattr(swa, "LIB_PATH", str(tmp_path / "libswa.so"))
    monkeypatch.setattr(swa, "_lib", None)
    with pytest.raises(ImportError):
        swa.lib()
    with pytest.raises(ImportError):
        swa.swa_cache_pool_bytes(swa.make_config(21, 2, 32, sliding_window_size=2))
