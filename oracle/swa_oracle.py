"""Float64 CPU oracle for frame-block sliding-window attention over a streaming KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The library under
``sliding_window_kv_amd`` never imports it and shares no code with it.

Everything here is plain NumPy in float64, written to be checked by eye
against the pages:

* "Sliding Window Attention Mechanism in AggregatorStream: Implementation and
  Configuration Guide" (instagit.com) -- sections "Mask Generation in
  CausalAttention", "KV Cache Eviction Strategy", "Manual Sliding-Window Mask
  Construction", "Cache Reset Between Sequences" and its FAQ.
* "Stream.py Aggregator Input and Output Formats: A Complete Technical Guide"
  (instagit.com) -- "Positional Embeddings" (3-D RoPE as complex values of
  size head_dim/2).
* The sliding-window-attention explainer on akshathtiwari.co.in (its
  rolling-buffer and receptive-field paragraph).
* The codehub.bot symbol page of ``FlashInferBlock.forward`` -- the
  streaming branch (keyframe: append, evict, attend; non-keyframe: append with
  eviction deferred, attend, roll back).

Readings where the pages are silent:
  frames are bidirectional inside and causal across; num_frame_per_block only
  scales the window; scale frames are visible to every later frame; the
  cache's window counts frames; window -1 means no window; softmax scale is
  1/sqrt(D); keys are ordered by ascending frame index; a non-keyframe sees
  the cached keyframes plus itself; special rows are retained in a FIFO of at
  most R entries; 3-D RoPE rotates interleaved pairs with a per-band ladder;
  the q and k norms are layer norms over head_dim with a per-feature weight
  and bias (epsilon 1e-5 unless given); token-level decode keeps a rolling
  buffer of W slots per sequence and maps query head h to kv head
  h // (Hq // Hkv).

Parity unpinned (no printed values on the pages; pinned only by the quoted
control flow and the readings above): non-keyframe visibility, cross-frame
special retention and its bound R, the 3-D RoPE layout relative to the
reference model's own rotary module, and the kind of the q/k norm (the pages
name it only).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

REGION_FRAME = 0
REGION_SPECIAL = 1


# ---------------------------------------------------------------------------
# Frame visibility and the explicit token mask
# ---------------------------------------------------------------------------

def window_frames(sliding_window_size: int, num_frame_per_block: int) -> Optional[int]:
    """Window length in frames, or None for "no window".

    Guide "Mask Generation in CausalAttention": the window spans
    sliding_window_size * num_frame_per_block frames ending at the current
    frame.  Its FAQ: a size of -1 switches the window off (full causal).
    """
    if sliding_window_size == -1:
        return None
    if sliding_window_size <= 0 or num_frame_per_block <= 0:
        raise ValueError("sliding_window_size must be -1 or positive")
    return sliding_window_size * num_frame_per_block


def frame_visibility(F: int, sliding_window_size: int, num_frame_per_block: int,
                     scale_frames: int) -> np.ndarray:
    """Boolean [F, F]: may a query of frame i see the keys of frame j?

    Guide "Mask Generation in CausalAttention": keys run from
    window_start = max(0, i - sliding_window_size*num_frame_per_block + 1)
    to the current frame i, and that sliding mask is ANDed with the causal
    mask.  Scale frames (the first `scale_frames`) are never evicted from the
    cache ("KV Cache Eviction Strategy"), so they are ORed into the window
    for every frame at or after them.
    """
    W = window_frames(sliding_window_size, num_frame_per_block)
    vis = np.zeros((F, F), dtype=bool)
    for i in range(F):
        start = 0 if W is None else max(0, i - W + 1)
        for j in range(F):
            causal = j <= i
            in_window = j >= start
            is_scale = j < scale_frames
            vis[i, j] = causal and (in_window or is_scale)
    return vis


def token_mask(F: int, P: int, sliding_window_size: int, num_frame_per_block: int,
               scale_frames: int) -> np.ndarray:
    """Boolean [F*P, F*P] token mask: M[q, k] = V(q // P, k // P).

    Frame of a token = its index floor-divided by the tokens per frame
    ("num_frames = N // frame_seqlen" in the mask section); whole row blocks
    share one frame's visibility (the manual mask example fills row block i
    up to the end of frame i).
    """
    vis = frame_visibility(F, sliding_window_size, num_frame_per_block, scale_frames)
    fq = np.arange(F * P) // P
    return vis[fq[:, None], fq[None, :]]


# ---------------------------------------------------------------------------
# Attention with an explicit mask
# ---------------------------------------------------------------------------

def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                     return_weights: bool = False):
    """Softmax attention with a boolean mask, in float64.

    q [Nq, H, D], k and v [Nk, H, D], mask [Nq, Nk] (True = visible).
    Per head: S = Q K^T / sqrt(D), masked entries set to -inf, softmax along
    each row (subtract the row max, exponentiate, divide by the row sum),
    O = A V.  This is what scaled_dot_product_attention with a boolean mask
    computes (mask section of the guide).  Returns (O [Nq, H, D],
    LSE [H, Nq]) where LSE is the natural log of the row's softmax
    denominator of the scaled scores.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, H, D = q.shape
    Nk = k.shape[0]
    assert k.shape == (Nk, H, D) and v.shape == (Nk, H, D)
    assert mask.shape == (Nq, Nk)
    if not mask.any(axis=1).all():
        raise ValueError("a query row sees no key")
    scale = 1.0 / math.sqrt(D)
    out = np.empty((Nq, H, D), dtype=np.float64)
    lse = np.empty((H, Nq), dtype=np.float64)
    weights = np.empty((H, Nq, Nk), dtype=np.float64) if return_weights else None
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) * scale
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        denom = e.sum(axis=1, keepdims=True)
        a = e / denom
        out[:, h, :] = a @ v[:, h, :]
        lse[h, :] = (m + np.log(denom))[:, 0]
        if return_weights:
            weights[h] = a
    if return_weights:
        return out, lse, weights
    return out, lse


def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, F: int, P: int,
            sliding_window_size: int, num_frame_per_block: int, scale_frames: int):
    """Masked prefill over F frames submitted at once ([F*P, H, D] each).

    One query row block (one frame) at a time against all keys with that
    block's rows of the explicit token mask; every row's arithmetic is the
    one in ``masked_attention``.
    """
    N = F * P
    if q.shape[0] != N:
        raise ValueError("token count is not F*P")
    H = q.shape[1]
    out = np.empty(q.shape, dtype=np.float64)
    lse = np.empty((H, N), dtype=np.float64)
    vis = frame_visibility(F, sliding_window_size, num_frame_per_block, scale_frames)
    fk = np.arange(N) // P
    for i in range(F):
        rows = slice(i * P, (i + 1) * P)
        mask = np.broadcast_to(vis[i][fk][None, :], (P, N))
        o, l = masked_attention(q[rows], k, v, mask)
        out[rows] = o
        lse[:, rows] = l
    return out, lse


# ---------------------------------------------------------------------------
# 3-D rotary embedding
# ---------------------------------------------------------------------------

def rope3d(x: np.ndarray, pos: np.ndarray, pairs_t: int, pairs_h: int, pairs_w: int,
           theta: float = 10000.0) -> np.ndarray:
    """Rotate interleaved pairs of x [N, H, D] by 3-D positions pos [N, 3].

    The guide's 3-D RoPE holds one complex value per pair, head_dim/2 of them
    per token.  Pair p is x[2p] + i*x[2p+1].  The pairs are split into a
    temporal, a height and a width band (in that order, sizes pairs_t,
    pairs_h, pairs_w).  Local pair kk of a band with d_b pairs turns by
    pos_b * theta**(-kk/d_b) radians (multiplication by exp(i*angle)).
    """
    x = np.asarray(x, dtype=np.float64)
    N, H, D = x.shape
    npairs = D // 2
    if pairs_t + pairs_h + pairs_w != npairs:
        raise ValueError("band sizes must add up to head_dim/2")
    angle = np.zeros((N, npairs), dtype=np.float64)
    p = 0
    for b, d_b in enumerate((pairs_t, pairs_h, pairs_w)):
        for kk in range(d_b):
            freq = float(theta) ** (-kk / d_b)
            angle[:, p] = pos[:, b].astype(np.float64) * freq
            p += 1
    z = x[..., 0::2] + 1j * x[..., 1::2]            # [N, H, D/2]
    z = z * np.exp(1j * angle)[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


# ---------------------------------------------------------------------------
# Per-head q/k normalisation
# ---------------------------------------------------------------------------

def head_layer_norm(x: np.ndarray, weight: np.ndarray, bias: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """Normalise every (token, head) row of x [N, H, D] over head_dim.

    The streaming branch's pre-attention pass names a q norm and a k norm
    between the reshape to heads and RoPE (codehub.bot, FlashInferBlock.forward,
    the compiled pre-attention step) but not their kind.  Read as a layer
    norm over the D features of one head: subtract the row mean, divide by
    sqrt(biased variance + eps), then scale by weight[d] and add bias[d]
    (weight and bias of length D, shared by all heads and tokens).
    """
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + float(eps)) * np.asarray(weight, np.float64) + np.asarray(bias, np.float64)


# ---------------------------------------------------------------------------
# Token-level decode over a rolling buffer (grouped-query heads)
# ---------------------------------------------------------------------------

class RollingDecodeCache:
    """Per-sequence rolling buffer of W slots (the explainer's decode cache).

    The key and value of the token at position i are written to slot i mod W,
    overwriting position i - W, which no later query can see: a query at
    position i attends itself and the W - 1 positions before it.  With
    grouped-query attention, query head h reads kv head h // (Hq // Hkv).
    Plain lists of float64 arrays; the slot arithmetic is kept only to report
    where each position lives.
    """

    def __init__(self, W: int, Hkv: int, D: int):
        if W < 1:
            raise ValueError("window must be >= 1")
        self.W, self.Hkv, self.D = W, Hkv, D
        self.slots = [None] * W            # slot -> (position, k [Hkv, D], v [Hkv, D])

    def append(self, pos: int, k: np.ndarray, v: np.ndarray) -> int:
        s = pos % self.W
        self.slots[s] = (pos, np.asarray(k, np.float64), np.asarray(v, np.float64))
        return s

    def attend(self, pos: int, q: np.ndarray):
        """q [Hq, D] of the token at position pos -> (out [Hq, D], lse [Hq])."""
        q = np.asarray(q, np.float64)
        Hq = q.shape[0]
        G = Hq // self.Hkv
        live = [e for e in self.slots if e is not None and pos - self.W < e[0] <= pos]
        assert live, "the current token is always visible"
        live.sort(key=lambda e: e[0])
        K = np.stack([e[1] for e in live])             # [n, Hkv, D]
        V = np.stack([e[2] for e in live])
        out = np.empty((Hq, self.D))
        lse = np.empty(Hq)
        for h in range(Hq):
            g = h // G
            s = K[:, g, :] @ q[h] / math.sqrt(self.D)
            m = s.max()
            w = np.exp(s - m)
            out[h] = w @ V[:, g, :] / w.sum()
            lse[h] = m + math.log(w.sum())
        return out, lse


# ---------------------------------------------------------------------------
# Naive ring cache
# ---------------------------------------------------------------------------

@dataclass
class CacheConfig:
    P: int
    sliding_window_size: int = -1
    num_frame_per_block: int = 1
    scale_frames: int = 0
    cross_frame_special: bool = False
    special_row0: int = 0
    special_rows: int = 5
    max_special_frames: int = 1000
    max_frames: int = 64          # capacity when the window is off

    @property
    def W(self) -> Optional[int]:
        return window_frames(self.sliding_window_size, self.num_frame_per_block)

    @property
    def scratch_slot(self) -> int:
        return self.max_frames if self.W is None else self.scale_frames + self.W


@dataclass
class _Entry:
    frame: int
    slot: int
    k: np.ndarray
    v: np.ndarray


@dataclass
class _Special:
    frame: int
    index: int                    # push count at the time it was retained
    k: np.ndarray
    v: np.ndarray


class RingError(RuntimeError):
    pass


class NaiveRingCache:
    """Per-layer rolling cache of whole frames, stored by value.

    Steps follow the streaming branch of ``FlashInferBlock.forward``:
    keyframe = append, evict, attend; non-keyframe = append with eviction
    deferred, attend, roll back.  Eviction is the guide's rule: when more
    than window + scale frames are cached, drop cached positions
    [scale_frames, n_cached - window).  Slots are bookkeeping only (data is
    held by value): scale frame n sits in slot n, the window is a rolling
    buffer written at slot scale_frames + ((n - scale_frames) mod window) for
    keyframe ordinal n (the explainer's "slot i modulo W" rule, shifted past
    the scale slots), a pending non-keyframe uses the slot after the window.
    """

    def __init__(self, cfg: CacheConfig):
        self.cfg = cfg
        self.reset()

    def reset(self):
        self.cached: List[_Entry] = []
        self.specials: List[_Special] = []
        self.n_key = 0
        self.n_special_pushed = 0
        self.pending: Optional[_Entry] = None
        self.last_frame: Optional[int] = None

    # -- state changes -----------------------------------------------------
    def append(self, t: int, k: np.ndarray, v: np.ndarray, keyframe: bool = True):
        cfg = self.cfg
        if self.pending is not None:
            raise RingError("a non-keyframe is pending; roll it back first")
        if t < 0 or (self.last_frame is not None and t <= self.last_frame):
            raise RingError("frame indices must be non-negative and increase")
        W, S = cfg.W, cfg.scale_frames
        if W is not None and len(self.cached) > S + W:
            raise RingError("evict before the next append")
        if keyframe:
            n = self.n_key
            if W is None:
                if n >= cfg.max_frames:
                    raise RingError("capacity")
                slot = n
            elif n < S:
                slot = n
            else:
                slot = S + (n - S) % W
            self.n_key += 1
            self.cached.append(_Entry(t, slot, np.array(k, np.float64), np.array(v, np.float64)))
        else:
            self.pending = _Entry(t, cfg.scratch_slot, np.array(k, np.float64),
                                  np.array(v, np.float64))
        self.last_frame = t

    def evict(self):
        cfg = self.cfg
        W, S = cfg.W, cfg.scale_frames
        if W is None or self.pending is not None:
            return []                      # window off, or eviction deferred
        n_cached = len(self.cached)
        if n_cached <= W + S:
            return []
        victims = self.cached[S:n_cached - W]
        self.cached = self.cached[:S] + self.cached[n_cached - W:]
        if cfg.cross_frame_special:
            r0, ns = cfg.special_row0, cfg.special_rows
            for vct in victims:
                self.specials.append(_Special(vct.frame, self.n_special_pushed,
                                              vct.k[r0:r0 + ns].copy(), vct.v[r0:r0 + ns].copy()))
                self.n_special_pushed += 1
            while len(self.specials) > cfg.max_special_frames:
                self.specials.pop(0)
        return [vct.frame for vct in victims]

    def rollback(self):
        if self.pending is None:
            raise RingError("nothing to roll back")
        self.pending = None

    # -- views ---------------------------------------------------------------
    def _ordered(self):
        """(record, k rows, v rows) in key order: scale, specials, window, pending."""
        cfg = self.cfg
        S = cfg.scale_frames if cfg.W is not None else len(self.cached)
        out = []
        for e in self.cached[:S]:
            out.append(((e.frame, REGION_FRAME, e.slot, 0, cfg.P), e.k, e.v))
        R, ns = cfg.max_special_frames, cfg.special_rows
        for s in self.specials:
            slot = s.index % R
            out.append(((s.frame, REGION_SPECIAL, slot, slot * ns, ns), s.k, s.v))
        for e in self.cached[S:]:
            out.append(((e.frame, REGION_FRAME, e.slot, 0, cfg.P), e.k, e.v))
        if self.pending is not None:
            e = self.pending
            out.append(((e.frame, REGION_FRAME, e.slot, 0, cfg.P), e.k, e.v))
        return out

    def visible_pages(self):
        """Page records (frame, region, slot, row0, nrows) in key order."""
        return [rec for rec, _, _ in self._ordered()]

    def keys_values(self):
        od = self._ordered()
        k = np.concatenate([kk for _, kk, _ in od])
        v = np.concatenate([vv for _, _, vv in od])
        return k, v

    def attend(self, q: np.ndarray):
        """Attention of q [P, H, D] over every cached key (all are visible).

        The guide's "KV Cache Eviction Strategy" evicts before attention, so
        a keyframe appended to a full window must be followed by evict()
        before attend(): in between, more than window + scale frames are
        cached and attending is refused.
        """
        W, S = self.cfg.W, self.cfg.scale_frames
        if W is not None and len(self.cached) > S + W:
            raise RingError("evict before attending")
        k, v = self.keys_values()
        mask = np.ones((q.shape[0], k.shape[0]), dtype=bool)
        return masked_attention(q, k, v, mask)

    # -- one streaming step ----------------------------------------------------
    def step(self, t: int, q: np.ndarray, k: np.ndarray, v: np.ndarray,
             keyframe: bool = True):
        """One layer's streaming step; returns (out, lse, page records used)."""
        if keyframe:
            self.append(t, k, v, True)
            self.evict()
            pages = self.visible_pages()
            out, lse = self.attend(q)
        else:
            self.append(t, k, v, False)
            pages = self.visible_pages()
            out, lse = self.attend(q)
            self.rollback()
        return out, lse, pages


def stream_replay(cfg: CacheConfig, frames, steps: int, keyframe_of=lambda t: True, pos_of=None,
                  rope_pairs=None, theta: float = 10000.0, record=None, rows=None, store=None):
    """Feed frames 0 .. steps-1 through one layer's NaiveRingCache, one per step.

    A generator.  frames(t) -> (q, k, v), each [P, H, D], for frame t.  Each
    step follows the streaming branch of FlashInferBlock.forward: a keyframe
    appends, evicts and attends; a non-keyframe (keyframe_of(t) false)
    appends with eviction deferred, attends and rolls back.  With pos_of(t)
    -> int [P, 3] and rope_pairs = (pairs_t, pairs_h, pairs_w), k is rotated
    by rope3d before it enters the cache and q before it attends (the
    block's pre-attention step rotates both before caching and attention).
    store, if given, is applied to the rotated q and k: it models the
    precision of the tensors that hold them (the rotation itself stays
    exact).

    Yields (t, pages, out, lse) per step: the visible-page records the step
    attended over and, for steps in `record` (every step if None), the
    attention output [n, H, D] and LSE [H, n] of query rows `rows` (all P
    rows if None); otherwise out and lse are None.
    """
    cache = NaiveRingCache(cfg)
    for t in range(steps):
        q, k, v = frames(t)
        keyframe = bool(keyframe_of(t))
        pos = pos_of(t) if pos_of is not None else None
        if pos is not None:
            k = rope3d(k, pos, *rope_pairs, theta=theta)
            if store is not None:
                k = store(k)
        cache.append(t, k, v, keyframe)
        if keyframe:
            cache.evict()
        pages = cache.visible_pages()
        out = lse = None
        if record is None or t in record:
            sel = slice(None) if rows is None else rows
            qs = q[sel]
            if pos is not None:
                qs = rope3d(qs, pos[sel], *rope_pairs, theta=theta)
                if store is not None:
                    qs = store(qs)
            out, lse = cache.attend(qs)
        if not keyframe:
            cache.rollback()
        yield t, pages, out, lse
