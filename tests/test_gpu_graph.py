"""GPU parity of the captured multi-layer streaming step (swa_graph_*), through
the C ABI: every replay of the graph is compared bit for bit with the same
frame stepped layer by layer through swa_stream_step(_normed) on a second
cache (same kernels, same work split), and with the float64 oracle (all rows
on small shapes, sampled rows at the 1374-token frame shape)."""
import numpy as np
import pytest
import torch

import sliding_window_kv_amd as swa
from gpu_helpers import assert_close_bf16, bf16_round_f64, case, dev, host, lse_tol
from oracle import CacheConfig, NaiveRingCache, head_layer_norm, rope3d
from swa_synth import frame_positions, frame_qkv, norm_weights

pytestmark = pytest.mark.gpu

EPS = 1e-5


def _oracle_step(oc, t, q, k, v, keyframe, rows):
    """One oracle step attending only the query rows `rows` (None: all)."""
    oc.append(t, k, v, keyframe)
    if keyframe:
        oc.evict()
    pages = oc.visible_pages()
    out, lse = oc.attend(q if rows is None else q[rows])
    if not keyframe:
        oc.rollback()
    return out, lse, pages


def _run(P, H, D, W, S, L, T, keyframe_of=lambda t: True, cross=False, ns=5, R=1000, rope=(0, 0, 0),
         grid=None, norm=False, rows=None, oracle_at=None, splits=None, sr0=0):
    cfg = swa.make_config(P, H, D, sliding_window_size=W, scale_frames=S, num_layers=L, cross_frame_special=cross,
                          special_row0=sr0, special_rows=ns, max_special_frames=R, rope=rope)
    gcache, ecache = swa.SwaCache(cfg), swa.SwaCache(cfg)
    if splits is not None:                   # before the capture: the column count is fixed in the graph
        gcache.set_splits(splits)
        ecache.set_splits(splits)
    qs = [torch.empty((P, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    ks = [torch.empty_like(qs[0]) for _ in range(L)]
    vs = [torch.empty_like(qs[0]) for _ in range(L)]
    outs = [torch.empty_like(qs[0]) for _ in range(L)]
    lses = [torch.empty((H, P), dtype=torch.float32, device="cuda") for _ in range(L)]
    posbuf = torch.empty((P, 3), dtype=torch.int32, device="cuda") if any(rope) else None
    ws = [norm_weights(60 + l, D) for l in range(L)]
    wds = [torch.from_numpy(w).cuda() for w in ws] if norm else None
    graph = swa.SwaGraph(gcache, qs, ks, vs, outs, lses, pos=posbuf, norm_weights=wds, eps=EPS)
    ocs = [NaiveRingCache(CacheConfig(P=P, sliding_window_size=W, scale_frames=S, cross_frame_special=cross,
                                      special_row0=sr0, special_rows=ns, max_special_frames=R)) for _ in range(L)]
    for t in range(T):
        kf = keyframe_of(t)
        frames = [frame_qkv(200 + l, t, P, H, D) for l in range(L)]
        pos = frame_positions(t, grid[0], grid[1], P - grid[0] * grid[1]) if any(rope) else None
        for l, (q, k, v) in enumerate(frames):
            qs[l].copy_(dev(q))
            ks[l].copy_(dev(k))
            vs[l].copy_(dev(v))
        if posbuf is not None:
            posbuf.copy_(torch.from_numpy(pos))
        graph.step(t, kf)
        pe = torch.from_numpy(pos).cuda() if pos is not None else None
        for l, (q, k, v) in enumerate(frames):
            qe, ke, ve = dev(q), dev(k), dev(v)
            oe = torch.empty_like(qe)
            le = torch.empty((H, P), dtype=torch.float32, device="cuda")
            if norm:
                ecache.step_normed(l, t, qe, ke, ve, wds[l], EPS, kf, oe, le, pos=pe)
            else:
                ecache.step(l, t, qe, ke, ve, kf, oe, le, pos=pe)
            torch.cuda.synchronize()
            assert torch.equal(outs[l], oe), f"out layer {l} t={t}"
            assert torch.equal(lses[l], le), f"lse layer {l} t={t}"
            assert torch.equal(qs[l], qe), f"q in place layer {l} t={t}"
            # the oracle sees the pre-attention pass in exact arithmetic, the
            # cached keys rounded to bf16 as the cache holds them
            qn, kn = q.astype(np.float64), k.astype(np.float64)
            if norm:
                qn = head_layer_norm(qn, ws[l][0], ws[l][1], EPS)
                kn = head_layer_norm(kn, ws[l][2], ws[l][3], EPS)
            if any(rope):
                qn, kn = rope3d(qn, pos, *rope), rope3d(kn, pos, *rope)
            if norm or any(rope):
                qn, kn = bf16_round_f64(qn), bf16_round_f64(kn)
            if oracle_at is None or t in oracle_at:
                ro, rl, pages = _oracle_step(ocs[l], t, qn, kn, v, kf, rows)
                got = host(outs[l]) if rows is None else host(outs[l])[rows]
                gl = host(lses[l]) if rows is None else host(lses[l])[:, rows]
                assert_close_bf16(got, ro, f"oracle layer {l} t={t}")
                assert np.abs(gl - rl).max() <= lse_tol(sum(p[4] for p in pages)), f"lse layer {l} t={t}"
                # after the step (a non-keyframe is rolled back again)
                assert gcache.pages(l) == [tuple(p) for p in ocs[l].visible_pages()], f"pages layer {l} t={t}"
            else:
                ocs[l].append(t, kn, v, kf)
                if kf:
                    ocs[l].evict()
                else:
                    ocs[l].rollback()
    for l in range(L):
        dp, n = gcache.device_pages(l)
        assert dp == gcache.pages(l) == ecache.pages(l), f"device pages layer {l}"
    graph.close()


@pytest.mark.parametrize("D", [64, 32])
def test_graph_small_all_rows(D):
    case(f"graph step P=200 H=4 D={D} W=4 S=2, 3 layers, 12 frames")
    _run(200, 4, D, 4, 2, 3, 12)


@pytest.mark.parametrize("splits", [1, 5])
def test_graph_fixed_splits(splits):
    # one piece per head (no merge launched), and five pieces per head: 20
    # columns, more than the 16 (head, tile) units of the first frame, so the
    # device clamps the column count as the per-layer path does on the host
    case(f"graph step with {splits} pieces per head")
    _run(200, 4, 64, 4, 2, 2, 9, splits=splits)


def test_graph_specials_nonkeyframes_rope_norm():
    # special rows retained into a 4-entry ring (wraps), every third frame a
    # non-keyframe, 3-D RoPE positions rewritten per frame, fused q/k norm
    case("graph step with retention, non-keyframes, rope and norm")
    _run(105, 2, 64, 3, 2, 2, 20, keyframe_of=lambda t: t % 3 != 2, cross=True, ns=5, R=4,
         rope=(12, 10, 10), grid=(10, 10), norm=True)


def test_graph_specials_across_tile_boundaries():
    # retention read from the device step plan, with the special rows
    # (60..68) straddling the append's 64-row work-group boundary in slot 0
    case("graph step with special rows 60..68, no scale frame")
    _run(150, 2, 64, 2, 0, 2, 12, keyframe_of=lambda t: t % 3 != 2, cross=True, ns=9, R=3, sr0=60)


def test_graph_frame_shape_sampled():
    # 1374-token frames, 16 heads, window 16 + 8 scale frames, two layers,
    # 30 frames (steady state from frame 24); every replay bit-exact against
    # the per-layer steps, sampled rows against the oracle at the end.
    P = 1374
    rows = np.array([0, 1, 31, 32, 63, 64, 127, 128, 700, 1279, 1280, 1343, 1344, 1373])
    case("graph step P=1374 H=16 D=64 W=16 S=8, 2 layers, 30 frames")
    _run(P, 16, 64, 16, 8, 2, 30, rows=rows, oracle_at={5, 29})


def test_graph_refuses_diverged_layers():
    P, H, D = 64, 2, 64
    case("graph step state checks")
    cfg = swa.make_config(P, H, D, sliding_window_size=2, scale_frames=1, num_layers=2)
    c = swa.SwaCache(cfg)
    bufs = [[torch.zeros((P, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(2)] for _ in range(4)]
    g = swa.SwaGraph(c, *bufs)
    g.step(0, True)
    k = torch.zeros((P, H, D), dtype=torch.bfloat16, device="cuda")
    c.append(0, 1, k, k)                     # layer 0 only
    with pytest.raises(swa.SwaError) as e:
        g.step(2, True)
    assert e.value.code == swa.SWA_E_STATE
    with pytest.raises(swa.SwaError) as e:
        swa.SwaGraph(c, *bufs)
    assert e.value.code == swa.SWA_E_STATE
    c.reset()                                # both layers empty again
    g.step(3, True)
    torch.cuda.synchronize()
    assert c.pages(0) == c.pages(1) == [(3, swa.SWA_REGION_FRAME, 0, 0, P)]
    g.close()


def test_graph_window_off_capacity():
    # window off: every keyframe stays (slot = ordinal) up to max_frames,
    # then the step is refused before anything is enqueued
    P, H, D = 96, 2, 64
    case("graph step, window off, capacity")
    cfg = swa.make_config(P, H, D, sliding_window_size=-1, max_frames=3, num_layers=2)
    gc, ec = swa.SwaCache(cfg), swa.SwaCache(cfg)
    q = [torch.empty((P, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    k = [torch.empty_like(q[0]) for _ in range(2)]
    v = [torch.empty_like(q[0]) for _ in range(2)]
    o = [torch.empty_like(q[0]) for _ in range(2)]
    g = swa.SwaGraph(gc, q, k, v, o)
    for t in range(4):
        kf = t != 1                              # frame 1 a non-keyframe: it is not kept
        frames = [frame_qkv(300 + l, t, P, H, D) for l in range(2)]
        for l, (a, b, c) in enumerate(frames):
            q[l].copy_(dev(a))
            k[l].copy_(dev(b))
            v[l].copy_(dev(c))
        g.step(t, kf)
        for l, (a, b, c) in enumerate(frames):
            oe = torch.empty_like(o[l])
            ec.step(l, t, dev(a), dev(b), dev(c), kf, oe, None)
            torch.cuda.synchronize()
            assert torch.equal(o[l], oe), f"out layer {l} t={t}"
    assert [p[0] for p in gc.pages(0)] == [0, 2, 3]
    with pytest.raises(swa.SwaError) as e:
        g.step(4, True)
    assert e.value.code == swa.SWA_E_CAPACITY
    assert gc.pages(1) == ec.pages(1)            # nothing advanced on the refused step
    g.close()
