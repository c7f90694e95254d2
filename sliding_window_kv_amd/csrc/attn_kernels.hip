// Frame-block sliding-window attention on gfx950.
//
// What is computed (guide "Sliding Window Attention Mechanism in
// AggregatorStream", sections "Mask Generation in CausalAttention" and "KV
// Cache Eviction Strategy"): for each head and query row,
//   O = sum_k softmax_k(q.k / sqrt(D)) v_k
// over the visible keys only.  Eviction happens before attention, so the
// streaming kernel walks exactly the rows of the visible pages; the prefill
// kernel walks exactly the visible key frames of the query tile's frame.
// Invisible keys are never loaded (whole tiles are skipped, not masked).
//
// bf16 kernel design (CDNA4, wave64):
//  * A work-group of NW waves owns NW*QB*32 query rows of one frame and head.
//    Each wave holds Q^T for QB blocks of 32 queries in registers as the B
//    operand of v_mfma_f32_32x32x16_bf16.
//  * Keys stream through LDS in 64-aligned tiles of 64 rows, in a ring of
//    kRing buffers (kRing - 1 tiles in flight while one is consumed), loaded
//    with direct buffer->LDS 16-byte loads (no staging registers).  A tile
//    is a contiguous 64 x D block of K rows and, with V^T stored in blocks of
//    64 keys, a contiguous [D][64] block of V^T; in LDS both are kept in that
//    shape with 16-byte chunks XOR-swizzled by row, so the MFMA operand reads
//    are free of bank conflicts.
//  * S^T = K Q^T: the accumulator layout puts one query per lane column and
//    16 keys per lane, so a query's row max needs one cross-half exchange
//    and the row sum stays lane-local until the end.
//  * The exponentiated scores are converted to bf16 in registers and used
//    directly as the B operand of O^T = V^T P^T: the key order inside each
//    16-key step follows the accumulator layout, and V^T is stored with that
//    order (vt_pos), so each lane's A operand is one 16-byte LDS read.
//  * Offset softmax in the log2 domain (scores scaled by log2(e)/sqrt(D)):
//    each query keeps one offset for its whole key range, the maximum of its
//    scores in the range's first tile, so later tiles need neither a running
//    maximum nor a rescale of O; with Q pre-scaled the offset enters the
//    score product's start value and P = 2^S costs one exponential per
//    score.  The row sum is taken over the bf16 probabilities the MFMA
//    consumes (v_dot2).  A range whose row sums leave the safe range (scores
//    spread too far for one offset) is recomputed with the running-max
//    softmax, which skips the O rescale when no lane's maximum moved.
//  * Segment edges: tiles start on a 64-row boundary; keys outside the
//    segment get score -inf and their V^T elements are cleared in LDS.
#include <math.h>

#include <algorithm>

#include "launch.hpp"

namespace swa {

namespace {

constexpr int KT = 64;            // keys per tile
constexpr int KALIGN = 64;        // tile start alignment (rows): one V^T block per tile
#ifndef SWA_RING
#define SWA_RING 3
#endif
constexpr int kRing = SWA_RING;   // K/V tile buffers in the ring
constexpr int kMaxBufs = 5;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int NW, int QB>
struct Shape {
    static constexpr int NT = NW * 64;
    static constexpr int QROWS = NW * QB * 32;
};

__device__ __forceinline__ int tiles_of(int lo, int hi) {
    const int b = lo & ~(KALIGN - 1);
    return (hi - b + KT - 1) / KT;
}

// The (at most two) key segments of a prefill query frame, kept in scalars.
struct PreSegs {
    int n, lo0, hi0, lo1, hi1, t1, total;
};

__device__ __forceinline__ PreSegs prefill_segs(int i, int W, int S, int fP) {
    int a0, a1, b0, b1;
    prefill_ranges(i, W, S, &a0, &a1, &b0, &b1);
    const bool has_a = a1 > a0;
    const bool has_b = b1 > b0;
    PreSegs s;
    // segment 0 is A when present, else B; segment 1 is B after A
    s.lo0 = has_a ? a0 * fP : b0 * fP;
    s.hi0 = has_a ? a1 * fP : b1 * fP;
    s.lo1 = b0 * fP;
    s.hi1 = b1 * fP;
    s.t1 = tiles_of(s.lo0, s.hi0);
    s.n = (has_a ? 1 : 0) + (has_b ? 1 : 0);
    s.total = s.t1 + (has_a && has_b ? tiles_of(s.lo1, s.hi1) : 0);
    return s;
}

// Segment accessors: streaming reads the list from kernel arguments (IND:
// from device memory, through the constant address space so the reads stay
// uniform scalar loads; the list does not change during a launch), prefill
// from the scalars above.
template <bool PREFILL, bool IND = false>
struct SegSrc {
    using CSeg = const __attribute__((address_space(4))) SegList;
    const AttnParams& p;
    PreSegs pre;
    __device__ const SegList& ks() const { return p.seg; }
    __device__ CSeg* ds() const { return (CSeg*)(p.dseg); }
    __device__ int n() const { return PREFILL ? pre.n : IND ? ds()->n : ks().n; }
    __device__ int total() const { return PREFILL ? pre.total : IND ? ds()->total_tiles : ks().total_tiles; }
    __device__ int lo(int j) const { return PREFILL ? (j == 0 ? pre.lo0 : pre.lo1) : IND ? ds()->lo[j] : ks().lo[j]; }
    __device__ int hi(int j) const { return PREFILL ? (j == 0 ? pre.hi0 : pre.hi1) : IND ? ds()->hi[j] : ks().hi[j]; }
    __device__ int tile0(int j) const { return PREFILL ? (j == 0 ? 0 : pre.t1) : IND ? ds()->tile0[j] : ks().tile0[j]; }
};

// Position of tile t inside the segment list.
struct Cursor {
    int seg, base, lo, hi;
};

template <class Src>
__device__ __forceinline__ Cursor cursor_at(const Src& s, int t) {
    Cursor c;
    c.seg = 0;
    const int n = s.n();
    for (int x = 1; x < n; ++x)
        if (s.tile0(x) <= t) c.seg = x;
    c.lo = s.lo(c.seg);
    c.hi = s.hi(c.seg);
    c.base = (c.lo & ~(KALIGN - 1)) + (t - s.tile0(c.seg)) * KT;
    return c;
}

template <class Src>
__device__ __forceinline__ void cursor_next(const Src& s, Cursor* c) {
    c->base += KT;
    if (c->base >= c->hi && c->seg + 1 < s.n()) {
        c->seg += 1;
        c->lo = s.lo(c->seg);
        c->hi = s.hi(c->seg);
        c->base = c->lo & ~(KALIGN - 1);
    }
}

// Logical work-item index with the blockIdx -> XCD round-robin undone, so
// that consecutive logical items (which share K/V tiles) land on one XCD
// and its L2.
__device__ __forceinline__ int xcd_remap(int b, int G) {
    constexpr int kXcd = 8;
    const int q = G / kXcd;
    const int r = G % kXcd;
    const int x = b % kXcd;
    const int j = b / kXcd;
    return x * q + (x < r ? x : r) + j;
}

// LDS tiles are rows of 16-byte chunks.  The LDS serves a 16-byte read for
// 16 lanes per cycle from 256 consecutive bytes (64 banks), so the chunk
// index is XOR-ed with the row's position in units of 256 bytes: 16 lanes
// reading 16 consecutive rows at one logical chunk hit 16 distinct slots.
template <int CPR>
__device__ __forceinline__ int lds_swz(int row) {
    return (row / (16 / CPR)) % CPR;
}

// Clear the V^T elements of keys outside [c.lo, c.hi) in a landed tile.
template <int D, int NT>
__device__ __forceinline__ void tile_clear_edges(uint16_t* vs, const Cursor& c, int tid) {
    // rare path: keep its per-thread addresses out of loop-invariant code
    // motion, which would hold one register per buffer and element
    asm volatile("" : "+v"(tid));
    for (int e = tid; e < D * KT; e += NT) {
        const int d = e / KT;
        const int pos = e % KT;                      // storage position in the tile
        const int key = c.base + vt_pos(pos);        // the key stored there
        if (key < c.lo || key >= c.hi) {
            const int kc = pos / 8;
            vs[d * KT + ((kc ^ lds_swz<8>(d)) * 8) + pos % 8] = 0;
        }
    }
}

// Exchange between the two 32-lane halves of a wave: after the swap, `a`
// holds the lower half's values in both halves and `b` the upper half's, so
// max(a, b) and a + b combine each lane with lane ^ 32.  Written as inline
// assembly with both registers read-write: the compiler's builtin for this
// instruction returned the same register for both results.  The leading
// s_nop covers the VALU-write -> permlane-read hazard.
// Lane l gets x of lanes l % 32 (lo) and l % 32 + 32 (hi).  Written as asm:
// the builtin, given one value for both operands, was folded as if the swap
// changed nothing.  Not volatile, so the scheduler may move it.
__device__ __forceinline__ void xhalf_swap(float x, float* lo, float* hi) {
    unsigned a = __builtin_bit_cast(unsigned, x);
    unsigned b = a;
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    *lo = __builtin_bit_cast(float, a);
    *hi = __builtin_bit_cast(float, b);
}

__device__ __forceinline__ float xhalf_max(float x) {
    float a, b;
    xhalf_swap(x, &a, &b);
    return fmaxf(a, b);
}

__device__ __forceinline__ float xhalf_sum(float x) {
    float a, b;
    xhalf_swap(x, &a, &b);
    return a + b;
}

// Epilogue of one work item: the normalised output and LSE (piece < 0), or
// the un-normalised partial (O, m, l) of a key range in slot `piece` of the
// work area, for the merge kernel.
template <int D, int QB, bool PREFILL>
__device__ __forceinline__ void write_out(const AttnParams& p, const f32x16 (&o)[QB][D / 32], const float (&m)[QB],
                                          const float (&l)[QB], int qrow0, int frame, int h, int piece, int l32,
                                          int hl) {
    constexpr int DB = D / 32;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = xhalf_sum(l[qb]);
        const int r = qrow0 + qb * 32 + l32;
        if (r >= p.nq) continue;
        if (piece < 0) {
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            const int64_t g = (static_cast<int64_t>(frame) * p.nq + r) * p.rs + h * p.hs;
            uint16_t* dst = static_cast<uint16_t*>(p.out) + g;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = db * 32 + 8 * g4 + 4 * hl;
                    const uint32_t w0 = pack_bf2(o[qb][db][4 * g4] * inv, o[qb][db][4 * g4 + 1] * inv);
                    const uint32_t w1 = pack_bf2(o[qb][db][4 * g4 + 2] * inv, o[qb][db][4 * g4 + 3] * inv);
                    *reinterpret_cast<u32x2*>(dst + d) = u32x2{w0, w1};
                }
            if (p.lse != nullptr && hl == 0)
                p.lse[static_cast<size_t>(h) * p.nq * (PREFILL ? p.F : 1) + static_cast<size_t>(frame) * p.nq + r] =
                    (m[qb] + log2f(lt)) * 0.69314718055994530942f;
        } else {
            const size_t row = static_cast<size_t>(piece) * p.nq + r;
            float* dst = p.part_o + row * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = db * 32 + 8 * g4 + 4 * hl;
                    *reinterpret_cast<f32x4*>(dst + d) =
                        f32x4{o[qb][db][4 * g4], o[qb][db][4 * g4 + 1], o[qb][db][4 * g4 + 2], o[qb][db][4 * g4 + 3]};
                }
            if (hl == 0) {
                p.part_ml[row * 2] = m[qb];
                p.part_ml[row * 2 + 1] = lt;
            }
        }
    }
}

// Per-lane byte offsets of the 16-byte chunks a thread loads into one K
// tile ([64][D], swizzled) and one V^T tile ([D][64], swizzled) from the
// tile's K rows and V^T block, each contiguous and starting at element
// base * D of its head's region: every load is that uniform offset plus one
// of these constant ones.
template <int D, int NW>
struct TileOffsets {
    static constexpr int CPR = D / 8;
    static constexpr int NK = KT * CPR / (64 * NW);
    static constexpr int NV = D * (KT / 8) / (64 * NW);
    int k[NK];
    int v[NV];
    __device__ TileOffsets(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int p = (i * NW + wave) * 64 + lane;
            const int row = p / CPR;
            k[i] = (row * D + ((p % CPR) ^ lds_swz<CPR>(row)) * 8) * 2;
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int p = (i * NW + wave) * 64 + lane;
            const int d = p / 8;
            v[i] = (d * KT + ((p % 8) ^ lds_swz<8>(d)) * 8) * 2;
        }
    }
};

// Direct buffer->LDS loads of the 64-key tile starting at row `base`.
template <int D, int NW>
__device__ __forceinline__ void tile_load(const TileOffsets<D, NW>& off, __amdgpu_buffer_rsrc_t kh, __amdgpu_buffer_rsrc_t vh,
                                          int base, uint16_t* ks, uint16_t* vs, int wave) {
    using TO = TileOffsets<D, NW>;
    // buffer loads: the tile's byte offset in a scalar, the lane's in a
    // vector register, so no load needs 64-bit address arithmetic (which the
    // global form took per load)
    const uint32_t sb = static_cast<uint32_t>(base) * (D * 2u);
#pragma unroll
    for (int i = 0; i < TO::NK; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kh, (__attribute__((address_space(3))) void*)(ks + (i * NW + wave) * 512),
                                                 16, static_cast<uint32_t>(off.k[i]), sb, 0, 0);
#pragma unroll
    for (int i = 0; i < TO::NV; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vh, (__attribute__((address_space(3))) void*)(vs + (i * NW + wave) * 512),
                                                 16, static_cast<uint32_t>(off.v[i]), sb, 0, 0);
}

// The three phases of one 64-key tile for one wave.  LDS reads address a
// tile as slot base + per-lane part (+ a constant for the second 32-row
// half); the per-lane parts come precomputed (TileLanes), so a kernel with
// many slots does not keep one address register per slot and read.
template <int D>
struct TileLanes {
    static constexpr int KS = D / 16;
    int k[KS];               // K tile: row l32, chunk (2*ks + hl) ^ swizzle, in bytes
    int v[4];                // V^T tile: row l32, chunk (4*kb + 2*hf + hl) ^ swizzle, in bytes
    __device__ TileLanes(int l32, int hl) {
        constexpr int CPR = D / 8;
        const int ksw = lds_swz<CPR>(l32);
        const int vsw = lds_swz<8>(l32);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) k[ks] = (l32 * CPR + ((ks * 2 + hl) ^ ksw)) * 16;
#pragma unroll
        for (int x = 0; x < 4; ++x) v[x] = (l32 * KT + ((x * 2 + hl) ^ vsw) * 8) * 2;
    }
    // Hide the values from loop-invariant code motion: added to each slot's
    // constant base at the read, not hoisted as one register per slot.
    __device__ __forceinline__ void refresh() {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(k[ks]));
#pragma unroll
        for (int x = 0; x < 4; ++x) asm volatile("" : "+v"(v[x]));
    }
};

// Scores: S^T = K Q^T (MFMA; the accumulator of lane l, register i holds
// key 8*(i/4) + 4*(l/32) + i%4 of each 32-key half and query l%32).  The
// first k-step starts from zero (ZERO) or from init[qb], which the offset
// softmax uses to subtract each query's offset inside the product.
template <int D, int QB, bool ZERO>
__device__ __forceinline__ void tile_scores(const uint16_t* ks, const bf16x8 (&qf)[QB][D / 16], f32x16 (&s)[2][QB],
                                            const TileLanes<D>& tl, const f32x16 (&init)[QB]) {
    constexpr int KS = D / 16;
    const f32x16 zero16 = {};
#pragma unroll
    for (int ks_ = 0; ks_ < KS; ++ks_) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(ks + kb * 32 * D) + tl.k[ks_]);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8, a), qf[qb][ks_], ks_ == 0 ? (ZERO ? zero16 : init[qb]) : s[kb][qb], 0,
                    0, 0);
        }
    }
}

// Keys outside the tile's segment get score -inf (rare path: tiles at
// segment edges).
template <int QB>
__device__ __forceinline__ void tile_mask(f32x16 (&s)[2][QB], const Cursor& cur, int hl, int edge) {
    if (edge) {
        // its 32 per-lane key offsets must not be hoisted into registers
        // held across the whole loop
        int hx = hl;
        asm volatile("" : "+v"(hx));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = cur.base + kb * 32 + 8 * (i >> 2) + 4 * hx + (i & 3);
                if (key < cur.lo || key >= cur.hi) {
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[kb][qb][i] = -INFINITY;
                }
            }
    }
}

// Online softmax (vector ALUs): keys outside the tile's segment get -inf;
// new running max m (log2 domain), O and l rescaled when any lane's max
// moved; P = 2^(s*scale - m) rounded to bf16 into the B operand of the PV
// product, and l accumulates exactly those bf16 values.
template <int D, int QB>
__device__ __forceinline__ void tile_softmax(f32x16 (&s)[2][QB], const Cursor& cur, bf16x8 (&pb)[2][QB][2],
                                             f32x16 (&o)[QB][D / 32], float (&m)[QB], float (&l)[QB], float sl2,
                                             int hl, int edge) {
    constexpr int DB = D / 32;
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    tile_mask<QB>(s, cur, hl, edge);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float mx = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][qb][i]);
        mx = xhalf_max(mx);
        const float mnew = fmaxf(m[qb], mx * sl2);
        if (__builtin_amdgcn_ballot_w64(mnew > m[qb]) != 0) {
            const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha;
            l[qb] *= alpha;
        }
        m[qb] = mnew;
        float ls = l[qb];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][hf * 8 + 2 * e], sl2, -mnew));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][hf * 8 + 2 * e + 1], sl2, -mnew));
                    w[e] = pack_bf2(p0, p1);
                    ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, ls, false);
                }
                pb[kb][qb][hf] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
            }
        l[qb] = ls;
    }
}

// O^T += V^T P^T (MFMA); V^T rows hold keys in vt_pos order, so one 16-byte
// LDS read per lane is the A operand matching P's register layout.
template <int D, int QB>
__device__ __forceinline__ void tile_pv(const uint16_t* vs, const bf16x8 (&pb)[2][QB][2], f32x16 (&o)[QB][D / 32],
                                        const TileLanes<D>& tl) {
    constexpr int DB = D / 32;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x4 a =
                    *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(vs + db * 32 * KT) + tl.v[kb * 2 + hf]);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb[kb][qb][hf],
                                                                        o[qb][db], 0, 0, 0);
            }
}

// Offset softmax.  Softmax is unchanged by a per-query shift of the scores,
// so instead of a running maximum each query keeps one offset m for the
// whole key range: the maximum of its scores in the range's first tile.
// Q is pre-scaled by log2(e)/sqrt(D) (rounded to bf16), and the score
// product of every later tile starts from -m, so it yields s - m directly:
// per tile only P = 2^(s - m) (rounded to bf16 for the PV product), and the
// row sum l over those bf16 values remain on the vector ALUs.  Later scores
// may exceed m; P > 1 is fine while it stays far from overflow, which the
// caller checks on l at the end (l is at least 1 and below 2^64 unless the
// scores of the range spread by more than about 40 in log2 units) and
// otherwise recomputes the range with the running-max softmax.
template <int D, int QB>
struct Acc {
    bf16x8 qf[QB][D / 16];   // Q^T operands
    f32x16 o[QB][D / 32];    // O^T accumulators
    float m[QB], l[QB];      // running max or offset (log2 domain) and row sum, per lane
    f32x16 c0[QB];           // offset softmax: score accumulator start, -m of the lane's query
    int live;                // nonzero: the wave holds at least one query row (else it only loads and waits)
    int wave;                // the wave's index in the work-group (uniform)
};

enum TileMode { kOnline = 0, kFirst = 1, kOffset = 2 };

// P = 2^x as bf16 into the B operand of the PV product, with x = s (the
// offset already inside the score product) or x = s * sl2 - m (FMA, Q not
// pre-scaled); l accumulates exactly those bf16 values (v_dot2 against
// ones).
template <int QB, bool FMA>
__device__ __forceinline__ void tile_exp(const f32x16 (&s)[2][QB], bf16x8 (&pb)[2][QB][2], float (&l)[QB],
                                         const float (&m)[QB], float sl2) {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float ls = l[qb];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x0 = s[kb][qb][hf * 8 + 2 * e], x1 = s[kb][qb][hf * 8 + 2 * e + 1];
                    const float p0 = __builtin_amdgcn_exp2f(FMA ? fmaf(x0, sl2, -m[qb]) : x0);
                    const float p1 = __builtin_amdgcn_exp2f(FMA ? fmaf(x1, sl2, -m[qb]) : x1);
                    w[e] = pack_bf2(p0, p1);
                    ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, ls, false);
                }
                pb[kb][qb][hf] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
            }
        l[qb] = ls;
    }
}

// First tile of the offset softmax: m = the query's maximum scaled score
// of the tile (the tile holds at least one key of the range).  Pre-scaled
// Q (PRE): the scores are shifted by m here and the accumulator start block
// -m serves the later tiles; otherwise each tile's exponent is one FMA.
template <int QB, bool PRE>
__device__ __forceinline__ void tile_first_offset(f32x16 (&s)[2][QB], float (&m)[QB], f32x16 (&c0)[QB], float sl2) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float mx = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][qb][i]);
        mx = xhalf_max(mx);
        if constexpr (PRE) {
            m[qb] = mx;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][qb][i] -= mx;
#pragma unroll
            for (int i = 0; i < 16; ++i) c0[qb][i] = -mx;
        } else {
            m[qb] = mx * sl2;
        }
    }
}


// One 64-key tile for one wave: scores, softmax (running max, or offset),
// PV product.  PRE: the offset softmax with Q pre-scaled (offset inside the
// score product); otherwise Q exact and the exponent one FMA.
template <int D, int QB, int MODE, bool PRE>
__device__ __forceinline__ void tile_step(const uint16_t* ks, const uint16_t* vs, const Cursor& cur, Acc<D, QB>& a,
                                          float sl2, int l32, int hl, int edge) {
    f32x16 s[2][QB];
    bf16x8 pb[2][QB][2];
    const TileLanes<D> tl(l32, hl);
    if constexpr (MODE == kOnline) {
        tile_scores<D, QB, true>(ks, a.qf, s, tl, a.c0);
        tile_softmax<D, QB>(s, cur, pb, a.o, a.m, a.l, sl2, hl, edge);
    } else if constexpr (MODE == kFirst) {
        tile_scores<D, QB, true>(ks, a.qf, s, tl, a.c0);
        tile_mask<QB>(s, cur, hl, edge);
        tile_first_offset<QB, PRE>(s, a.m, a.c0, sl2);
        tile_exp<QB, !PRE>(s, pb, a.l, a.m, sl2);
    } else {
        tile_scores<D, QB, !PRE>(ks, a.qf, s, tl, a.c0);
        tile_mask<QB>(s, cur, hl, edge);
        tile_exp<QB, !PRE>(s, pb, a.l, a.m, sl2);
    }
    tile_pv<D, QB>(vs, pb, a.o, tl);
}

// Work-group barrier after this wave's LDS accesses and all but its N
// youngest vector-memory operations have completed (loads return in order,
// so the older direct-to-LDS tiles have landed).  Not __syncthreads(): its
// fences made the compiler wait for every load in flight, the prefetched
// tiles included.  The wait is the builtin, not inline assembly, so that
// the compiler's own wait counting knows the older tiles have landed and
// adds no wait for all loads before the next LDS reads.
template <int N>
__device__ __forceinline__ void sync_tiles() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // s_waitcnt vmcnt(N) expcnt(7) lgkmcnt(0): vmcnt in bits 3:0 and 15:14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);           // no instruction moves across the barrier
}

// K/V tile ring of NB buffers: tile t lives in buffer t % NB and is loaded
// NB - 1 iterations ahead of its use.  One iteration (buffer U = it % NB):
// wait for tile `it` (the NB - 2 younger tiles may stay in flight), barrier
// (publishes tile `it`, and every wave is done with tile it - 1, whose
// buffer is refilled next), clear its edge keys, start loading tile
// it + NB - 1, then compute.  U is a compile-time constant and every buffer
// is an LDS variable of its own, so the compiler can tell the buffer being
// read from the ones being loaded (with one array it waited for all loads).
// FULL: every tile this iteration waits for or loads exists, so the load is
// unconditional; loops of such iterations have no branch around a tile load,
// across which the compiler's wait counting would again fall back to
// waiting for all loads in flight.
template <int D, int NW, int QB, int NB, int U, int MODE, bool PRE, bool FULL = false, class Src>
__device__ __forceinline__ void ring_iter(int it, int ntiles, Cursor (&cq)[NB], Cursor& ld, const Src& segs,
                                          const TileOffsets<D, NW>& off, __amdgpu_buffer_rsrc_t kh, __amdgpu_buffer_rsrc_t vh,
                                          uint16_t* const (&kbuf)[kMaxBufs], uint16_t* const (&vbuf)[kMaxBufs],
                                          Acc<D, QB>& a, float sl2, int tid) {
    using TO = TileOffsets<D, NW>;
    constexpr int PER_TILE = TO::NK + TO::NV;    // load instructions per wave per tile
    constexpr int NXT = (U + NB - 1) % NB;
    const int lane = tid & 63;
    const int wave = a.wave;
    if (FULL || it + NB - 2 < ntiles)
        sync_tiles<(NB - 2) * PER_TILE>();
    else
        sync_tiles<0>();
    const Cursor cur = cq[U];
    uint16_t* kcur = kbuf[U];
    uint16_t* vcur = vbuf[U];
    // uniform flag in a scalar register (else it travels to the masking in
    // tile_step as a per-lane boolean)
    const int edge = ((cur.base - cur.lo) | (cur.hi - cur.base - KT)) >> 31;   // -1: an edge tile, 0: interior
    if (edge) {
        tile_clear_edges<D, NW * 64>(vcur, cur, tid);
        sync_tiles<63>();
    }
    if (FULL || it + NB - 1 < ntiles) {
        cursor_next(segs, &ld);
        cq[NXT] = ld;
        tile_load<D, NW>(off, kh, vh, ld.base, kbuf[NXT], vbuf[NXT], wave);
    }
    if (a.live) tile_step<D, QB, MODE, PRE>(kcur, vcur, cur, a, sl2, lane & 31, lane >> 5, edge);
}

template <int D, int NW, int QB, int NB, int U, int MODE, bool PRE, class Src>
__device__ __forceinline__ void ring_tail(int it, int ntiles, Cursor (&cq)[NB], Cursor& ld, const Src& segs,
                                          const TileOffsets<D, NW>& off, __amdgpu_buffer_rsrc_t kh, __amdgpu_buffer_rsrc_t vh,
                                          uint16_t* const (&kbuf)[kMaxBufs], uint16_t* const (&vbuf)[kMaxBufs],
                                          Acc<D, QB>& a, float sl2, int tid) {
    if constexpr (U < NB) {
        if (it < ntiles) {
            ring_iter<D, NW, QB, NB, U, MODE, PRE>(it, ntiles, cq, ld, segs, off, kh, vh, kbuf, vbuf, a, sl2, tid);
            ring_tail<D, NW, QB, NB, U + 1, MODE, PRE>(it + 1, ntiles, cq, ld, segs, off, kh, vh, kbuf, vbuf, a, sl2, tid);
        }
    }
}

template <int D, int NW, int QB, int NB, int U, int MODE, bool PRE, bool FULL, class Src>
__device__ __forceinline__ void ring_round(int it, int ntiles, Cursor (&cq)[NB], Cursor& ld, const Src& segs,
                                           const TileOffsets<D, NW>& off, __amdgpu_buffer_rsrc_t kh, __amdgpu_buffer_rsrc_t vh,
                                           uint16_t* const (&kbuf)[kMaxBufs], uint16_t* const (&vbuf)[kMaxBufs],
                                           Acc<D, QB>& a, float sl2, int tid) {
    if constexpr (U < NB) {
        ring_iter<D, NW, QB, NB, U, MODE, PRE, FULL>(it + U, ntiles, cq, ld, segs, off, kh, vh, kbuf, vbuf, a, sl2, tid);
        ring_round<D, NW, QB, NB, U + 1, MODE, PRE, FULL>(it, ntiles, cq, ld, segs, off, kh, vh, kbuf, vbuf, a, sl2, tid);
    }
}

// Token decode: the new token's key row and V^T column of buffer h into
// row p.dslot (the cache region is the kernel's own buffer: writable).
template <int D, int NW>
__device__ __forceinline__ void decode_token_write(const AttnParams& p, int h, int tid) {
    const uint16_t* k = static_cast<const uint16_t*>(p.dk) + static_cast<size_t>(h) * D;
    const uint16_t* v = static_cast<const uint16_t*>(p.dv) + static_cast<size_t>(h) * D;
    uint16_t* kr = static_cast<uint16_t*>(const_cast<void*>(p.kreg)) + (static_cast<size_t>(h) * p.rows + p.dslot) * D;
    uint16_t* vr = static_cast<uint16_t*>(const_cast<void*>(p.vreg)) + static_cast<size_t>(h) * D * p.rows;
    for (int d = tid; d < D; d += NW * 64) {
        kr[d] = k[d];
        vr[vt_elem(d, vt_pos(p.dslot), D)] = v[d];
    }
}

// Q^T operands of this wave's query blocks (rows past the frame: zero),
// multiplied by `scale` and rounded to bf16 when scale != 0.
template <int D, int QB>
__device__ __forceinline__ void load_q(const AttnParams& p, int frame, int h, int qrow0, int l32, int hl, float scale,
                                       bf16x8 (&qf)[QB][D / 16]) {
    constexpr int KS = D / 16;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int r = qrow0 + qb * 32 + l32;
        const bool ok = r < p.nq;
        const int64_t g = (static_cast<int64_t>(frame) * p.nq + (ok ? r : 0)) * p.rs + h * p.hs;
        const uint16_t* src = static_cast<const uint16_t*>(p.q) + g + hl * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 u = ok ? *reinterpret_cast<const u32x4*>(src + ks * 16) : u32x4{0u, 0u, 0u, 0u};
            if (scale != 0.f) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    u[j] = pack_bf2(__builtin_bit_cast(float, u[j] << 16) * scale,
                                    __builtin_bit_cast(float, u[j] & 0xffff0000u) * scale);
            }
            qf[qb][ks] = __builtin_bit_cast(bf16x8, u);
        }
    }
}

// One pass over key tiles [t_begin, t_begin + ntiles) of the segment list
// (ntiles >= 1): the running-max softmax (OFFSET = false) or the offset
// softmax (OFFSET = true; PRE: with Q pre-scaled).
template <int D, int NW, int QB, bool OFFSET, bool PRE, class Src>
__device__ __forceinline__ void run_pass(const AttnParams& p, const Src& segs, int frame, int h, int qrow0,
                                         int t_begin, int ntiles, const TileOffsets<D, NW>& off, __amdgpu_buffer_rsrc_t kh,
                                         __amdgpu_buffer_rsrc_t vh, uint16_t* const (&KB)[kMaxBufs],
                                         uint16_t* const (&VB)[kMaxBufs], Acc<D, QB>& a, int tid) {
    constexpr int NB = kRing;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS destinations stay scalar
    const int l32 = lane & 31;
    const int hl = lane >> 5;

    // prologue: tiles 0 .. NB-2 in flight
    Cursor cq[NB];
    Cursor ld = cursor_at(segs, t_begin);
#pragma unroll
    for (int u = 0; u < NB - 1; ++u) {
        if (u > 0) cursor_next(segs, &ld);
        cq[u] = ld;
        if (u < ntiles) tile_load<D, NW>(off, kh, vh, ld.base, KB[u], VB[u], wave);
    }

    load_q<D, QB>(p, frame, h, qrow0, l32, hl, OFFSET && PRE ? p.scale_log2 : 0.f, a.qf);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        a.m[qb] = -INFINITY;
        a.l[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) a.o[qb][db][i] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a.c0[qb][i] = 0.f;
    }
    const float sl2 = p.scale_log2;

    if constexpr (OFFSET) {
        ring_iter<D, NW, QB, NB, 0, kFirst, PRE>(0, ntiles, cq, ld, segs, off, kh, vh, KB, VB, a, sl2, tid);
        ring_tail<D, NW, QB, NB, 1, kOffset, PRE>(1, ntiles, cq, ld, segs, off, kh, vh, KB, VB, a, sl2, tid);
        int it = NB;
        // rounds whose loads all exist, then at most one round with guarded loads
        for (; it + 2 * NB - 1 <= ntiles; it += NB)
            ring_round<D, NW, QB, NB, 0, kOffset, PRE, true>(it, ntiles, cq, ld, segs, off, kh, vh, KB, VB, a, sl2, tid);
        for (; it + NB <= ntiles; it += NB)
            ring_round<D, NW, QB, NB, 0, kOffset, PRE, false>(it, ntiles, cq, ld, segs, off, kh, vh, KB, VB, a, sl2, tid);
        ring_tail<D, NW, QB, NB, 0, kOffset, PRE>(it, ntiles, cq, ld, segs, off, kh, vh, KB, VB, a, sl2, tid);
    } else {
        int it = 0;
        for (; it + 2 * NB - 1 <= ntiles; it += NB)
            ring_round<D, NW, QB, NB, 0, kOnline, false, true>(it, ntiles, cq, ld, segs, off, kh, vh, KB, VB, a, sl2, tid);
        for (; it + NB <= ntiles; it += NB)
            ring_round<D, NW, QB, NB, 0, kOnline, false, false>(it, ntiles, cq, ld, segs, off, kh, vh, KB, VB, a, sl2, tid);
        ring_tail<D, NW, QB, NB, 0, kOnline, false>(it, ntiles, cq, ld, segs, off, kh, vh, KB, VB, a, sl2, tid);
    }
}

// One work item: query tile `qt` of (frame, head h) against key tiles
// [t_begin, t_end) of the segment list, finished by write_out(piece).  The
// offset-softmax pass runs first (PRE: with Q pre-scaled); if any of the
// work-group's queries ends with a row sum that is not finite or not below
// 2^64 (its scores spread too far for one fixed offset), the whole
// work-group recomputes the item with the running-max softmax.  badw: one
// LDS flag per wave.
template <int D, int NW, int QB, bool PREFILL, bool IND, bool PRE>
__device__ __forceinline__ void attend_range(const AttnParams& p, const SegSrc<PREFILL, IND>& segs, int h, int frame,
                                             int qt, int t_begin, int t_end, int piece, uint16_t* const (&KB)[kMaxBufs],
                                             uint16_t* const (&VB)[kMaxBufs], int* badw, int tid) {
    using Sh = Shape<NW, QB>;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hl = lane >> 5;
    const int ntiles = t_end - t_begin;

    const uint16_t* kp = static_cast<const uint16_t*>(p.kreg) + static_cast<size_t>(h) * p.rows * D;
    const uint16_t* vp = static_cast<const uint16_t*>(p.vreg) + static_cast<size_t>(h) * D * p.rows;
    // one head's K rows and V^T blocks as raw buffer resources: stride 0,
    // the region's bytes as the record count, 32-bit data format (word 3)
    constexpr int kRawBuffer = 0x00020000;
    const __amdgpu_buffer_rsrc_t kh =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kp), 0, p.rows * D * 2, kRawBuffer);
    const __amdgpu_buffer_rsrc_t vh =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vp), 0, p.rows * D * 2, kRawBuffer);
    const TileOffsets<D, NW> off(wave, lane);

    if constexpr (!PREFILL && NW == 1) {
        // token decode (one-wave work-groups): the one work item whose range
        // holds the new slot's tile (the buffer's single segment starts at
        // row 0) writes the new token first; its stores complete before the
        // tile loads below
        if (p.dk != nullptr && p.dslot / KT >= t_begin && p.dslot / KT < t_end) {
            decode_token_write<D, NW>(p, h, tid);
            sync_tiles<0>();
        }
    }

    const int qrow0 = qt * Sh::QROWS + wave * QB * 32;
    Acc<D, QB> a;
    a.live = __builtin_amdgcn_readfirstlane(qrow0 < p.nq ? 1 : 0);
    a.wave = wave;   // waves past the frame's last row skip the arithmetic
    run_pass<D, NW, QB, true, PRE>(p, segs, frame, h, qrow0, t_begin, ntiles, off, kh, vh, KB, VB, a, tid);
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) bad = bad || !(a.l[qb] < 0x1p64f);
    const bool wbad = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (lane == 0) badw[wave] = wbad ? 1 : 0;
    sync_tiles<0>();                                 // every wave's flag, and every wave done with the tiles
    bool online = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) online = online || badw[w] != 0;
    if (online)
        run_pass<D, NW, QB, false, false>(p, segs, frame, h, qrow0, t_begin, ntiles, off, kh, vh, KB, VB, a, tid);

    write_out<D, QB, PREFILL>(p, a.o, a.m, a.l, qrow0, frame, h, piece, l32, hl);
}

// Work decomposition.  Prefill: one work item per (frame, head, query tile),
// ordered head-major with the frames of a head from last to first: an XCD
// (a run of consecutive logical work-groups) then holds neighbouring frames
// of the same head at once, which share most of their visible key frames
// (all scale frames and most of the window) through its L2, and within a
// head the frames that see the most keys start first.
// Streaming: every query of the frame sees the same key tiles, so the
// (head, key tile) space of H * n tiles is cut into p.ncols equal columns,
// and column c runs as p.qtiles work-groups, one per query tile, that walk
// the same K/V tiles at the same time (consecutive work-groups: one XCD and
// its L2).  A column's range may end and start inside heads; such pieces go
// to the work area as partials (slot 2c for the column's first head, 2c + 1
// for its last) and the merge kernel combines them.  With ncols near
// (work-groups the GPU holds) / qtiles, every work-group gets the same
// number of tiles and the launch finishes in one round.  IND (captured
// steps): the segments come from device memory and the launch has a fixed
// number of columns, of which the first min(ncols, H * n) work.  PRE: the
// offset softmax with Q pre-scaled, chosen when no LSE is requested (its
// bf16 rounding of the scaled Q shifts a query's LSE by up to about 2^-9 of
// its score magnitude, but leaves the output within bf16 noise).
template <int D, int NW, int QB, int OCC, bool PREFILL, bool IND, bool PRE>
__global__ __launch_bounds__(NW * 64, OCC) void attn_bf16_kernel(AttnParams p) {
    constexpr int NB = kRing;
    static_assert(NB >= 2 && NB <= kMaxBufs, "2 to 5 tile buffers");

    __shared__ __attribute__((aligned(16))) uint16_t K0[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t K1[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t K2[NB > 2 ? KT * D : 8];
    __shared__ __attribute__((aligned(16))) uint16_t K3[NB > 3 ? KT * D : 8];
    __shared__ __attribute__((aligned(16))) uint16_t K4[NB > 4 ? KT * D : 8];
    __shared__ __attribute__((aligned(16))) uint16_t V0[D * KT];
    __shared__ __attribute__((aligned(16))) uint16_t V1[D * KT];
    __shared__ __attribute__((aligned(16))) uint16_t V2[NB > 2 ? D * KT : 8];
    __shared__ __attribute__((aligned(16))) uint16_t V3[NB > 3 ? D * KT : 8];
    __shared__ __attribute__((aligned(16))) uint16_t V4[NB > 4 ? D * KT : 8];
    __shared__ int badw[NW];
    uint16_t* const KB[kMaxBufs] = {K0, K1, K2, K3, K4};
    uint16_t* const VB[kMaxBufs] = {V0, V1, V2, V3, V4};

    const int tid = threadIdx.x;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = L % p.qtiles;
    const int item = L / p.qtiles;
    if constexpr (PREFILL) {
        const int h = item / p.F;
        const int frame = p.F - 1 - item % p.F;
        const SegSrc<true> segs{p, prefill_segs(frame, p.W, p.S, p.fP)};
        attend_range<D, NW, QB, true, false, PRE>(p, segs, h, frame, qt, 0, segs.total(), -1, KB, VB, badw, tid);
    } else {
        const SegSrc<false, IND> segs{p, PreSegs{}};
        const int n = segs.total();
        const int64_t hn = static_cast<int64_t>(p.H) * n;
        const int ncols = IND ? static_cast<int>(hn < p.ncols ? hn : p.ncols) : p.ncols;
        if (IND && item >= ncols) return;            // the whole work-group: no barrier is left waiting
        int64_t f = hn * item / ncols;
        const int64_t f1 = hn * (item + 1) / ncols;
        bool first = true;
        while (f < f1) {
            const int h = static_cast<int>(f / n);
            const int64_t h0 = static_cast<int64_t>(h) * n;
            const int t0 = static_cast<int>(f - h0);
            const int t1 = static_cast<int>(f1 - h0 < n ? f1 - h0 : n);
            const int piece = (t0 == 0 && t1 == n) ? -1 : 2 * item + (first ? 0 : 1);
            if (!first) sync_tiles<0>();                 // every wave is done with the last range's tiles
            attend_range<D, NW, QB, false, IND, PRE>(p, segs, h, 0, qt, t0, t1, piece, KB, VB, badw, tid);
            f = h0 + t1;
            first = false;
        }
    }
}

// Merge of the streaming partials: for head h the columns c_lo .. c_hi cover
// its tiles, and column c holds its piece in slot 2c if head h is the first
// head of the column, else in slot 2c + 1.  Every column after c_lo starts
// inside head h, so only c_lo can hold h's piece in its second slot: one
// division per thread picks that slot (64-bit divisions are long
// instruction sequences on the GPU).
//   O = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,  M = max_c m_c.
// Heads that lie inside one column were written by the attention kernel.
__device__ __forceinline__ int column_of(int64_t x, int64_t hn, int ncols) {
    return static_cast<int>(((x + 1) * ncols + hn - 1) / hn) - 1;   // the c with start(c) <= x < start(c + 1)
}

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                    uint16_t* __restrict__ out, float* __restrict__ lse, int H, int nq,
                                                    int n, int ncols, int64_t rs, int64_t hs,
                                                    const int* __restrict__ dn) {
    constexpr int C = D / 4;
    if (dn != nullptr) {                             // captured step: tile count from device memory
        n = *dn;
        ncols = static_cast<int64_t>(H) * n < ncols ? H * n : ncols;
    }
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= H * nq * C) return;
    const int chunk = idx % C;
    const int r = (idx / C) % nq;
    const int h = idx / (C * nq);
    const int64_t hn = static_cast<int64_t>(H) * n;
    const int64_t a = static_cast<int64_t>(h) * n;
    const int c_lo = column_of(a, hn, ncols);
    const int c_hi = column_of(a + n - 1, hn, ncols);
    if (c_lo == c_hi) return;
    const int first = 2 * c_lo + (hn * c_lo / ncols >= a ? 0 : 1);
    // one pass with a running max (unrolled so that several pieces' loads
    // are in flight at once): M, Lsum and acc rescaled when M moves
    float M = -INFINITY;
    float Lsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int c = c_lo; c <= c_hi; ++c) {
        const int piece = c == c_lo ? first : 2 * c;
        const size_t row = static_cast<size_t>(piece) * nq + r;
        const float ms = part_ml[row * 2];
        const float ls = part_ml[row * 2 + 1];
        const f32x4 oc = *reinterpret_cast<const f32x4*>(part_o + row * D + chunk * 4);
        if (ms > M) {
            const float scale = __builtin_amdgcn_exp2f(M - ms);     // 0 while M = -inf
            Lsum *= scale;
            acc *= scale;
            M = ms;
        }
        const float w = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
        Lsum += w * ls;
        acc += w * oc;
    }
    const float inv = 1.f / Lsum;
    const int64_t g = r * rs + h * hs + chunk * 4;
    *reinterpret_cast<u32x2*>(out + g) =
        u32x2{pack_bf2(acc[0] * inv, acc[1] * inv), pack_bf2(acc[2] * inv, acc[3] * inv)};
    if (lse != nullptr && chunk == 0) lse[static_cast<size_t>(h) * nq + r] = (M + log2f(Lsum)) * 0.69314718055994530942f;
}

// Merge for few query rows and many pieces per head (token decode).  Each
// (row, 4-feature chunk) item gets 16 lanes of one wave, which split the
// head's pieces; a lane loads a batch of its pieces at once, folds them with
// its own maximum, and the 16 lanes then combine their (max, sum, output)
// triples through cross-lane exchanges: no LDS and no barrier, and for up
// to 128 pieces per head a single round of loads.
constexpr int kDecodeLanes = 16;            // lanes per item
constexpr int kDecodeBatch = 8;             // pieces per lane loaded at once

template <int D>
__global__ __launch_bounds__(256) void merge_decode_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           uint16_t* __restrict__ out, float* __restrict__ lse, int H,
                                                           int nq, int n, int ncols, int64_t rs, int64_t hs,
                                                           const int* __restrict__ dn) {
    constexpr int C = D / 4;
    constexpr int IPB = 256 / kDecodeLanes;          // items per work-group
    if (dn != nullptr) {                             // captured step: tile count from device memory
        n = *dn;
        ncols = static_cast<int64_t>(H) * n < ncols ? H * n : ncols;
    }
    const int items = nq * C;
    const int blocks_per_head = (items + IPB - 1) / IPB;
    const int h = blockIdx.x / blocks_per_head;
    const int item = (blockIdx.x % blocks_per_head) * IPB + threadIdx.x / kDecodeLanes;
    const int pl = threadIdx.x % kDecodeLanes;
    const int64_t hn = static_cast<int64_t>(H) * n;
    const int64_t a = static_cast<int64_t>(h) * n;
    const int c_lo = column_of(a, hn, ncols);
    const int c_hi = column_of(a + n - 1, hn, ncols);
    if (c_lo == c_hi) return;                       // whole head in one column: written by the attention kernel
    const int npc = c_hi - c_lo + 1;
    const int first = 2 * c_lo + (hn * c_lo / ncols >= a ? 0 : 1);   // see merge_kernel
    // lanes past the last item load item 0's data and take part in the
    // exchanges, but store nothing
    const bool ok = item < items;
    const int r = ok ? item / C : 0;
    const int chunk = ok ? item % C : 0;
    float M = -INFINITY;
    float Ls = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = pl; j0 < npc; j0 += kDecodeLanes * kDecodeBatch) {
        float ms[kDecodeBatch], ls[kDecodeBatch];
        f32x4 oc[kDecodeBatch];
#pragma unroll
        for (int u = 0; u < kDecodeBatch; ++u) {
            const int j = j0 + u * kDecodeLanes;
            if (j < npc) {
                const int piece = j == 0 ? first : 2 * (c_lo + j);
                const size_t row = static_cast<size_t>(piece) * nq + r;
                ms[u] = part_ml[row * 2];
                ls[u] = part_ml[row * 2 + 1];
                oc[u] = *reinterpret_cast<const f32x4*>(part_o + row * D + chunk * 4);
            } else {
                ms[u] = -INFINITY;
                ls[u] = 0.f;
                oc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        float mb = M;
#pragma unroll
        for (int u = 0; u < kDecodeBatch; ++u) mb = fmaxf(mb, ms[u]);
        if (mb > M) {
            const float scale = __builtin_amdgcn_exp2f(M - mb);     // 0 while M = -inf
            Ls *= scale;
            acc *= scale;
            M = mb;
        }
#pragma unroll
        for (int u = 0; u < kDecodeBatch; ++u) {
            const float w = ms[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[u] - M);
            Ls += w * ls[u];
            acc += w * oc[u];
        }
    }
    // the item's 16 lanes are consecutive: exchanges with lane ^ 8, 4, 2, 1
    float Mg = M;
#pragma unroll
    for (int off = kDecodeLanes / 2; off >= 1; off >>= 1) Mg = fmaxf(Mg, __shfl_xor(Mg, off));
    const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mg);
    Ls *= sc;
    acc *= sc;
#pragma unroll
    for (int off = kDecodeLanes / 2; off >= 1; off >>= 1) {
        Ls += __shfl_xor(Ls, off);
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] += __shfl_xor(acc[k], off);
    }
    if (ok && pl == 0) {
        const float inv = 1.f / Ls;
        const int64_t g = r * rs + h * hs + chunk * 4;
        *reinterpret_cast<u32x2*>(out + g) =
            u32x2{pack_bf2(acc[0] * inv, acc[1] * inv), pack_bf2(acc[2] * inv, acc[3] * inv)};
        if (lse != nullptr && chunk == 0)
            lse[static_cast<size_t>(h) * nq + r] = (Mg + log2f(Ls)) * 0.69314718055994530942f;
    }
}

// fp32 path: one thread per query row, exact online softmax in single
// precision on the vector ALUs (latency-bound tiny workloads).
template <int D, bool PREFILL>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnParams p) {
    const int h = blockIdx.y;
    const int frame = PREFILL ? static_cast<int>(blockIdx.z) : 0;
    const int r = blockIdx.x * 64 + threadIdx.x;
    if (r >= p.nq) return;
    PreSegs pre{};
    if constexpr (PREFILL) pre = prefill_segs(frame, p.W, p.S, p.fP);
    const SegSrc<PREFILL> segs{p, pre};
    const int64_t g = (static_cast<int64_t>(frame) * p.nq + r) * p.rs + h * p.hs;
    const float* qp = static_cast<const float*>(p.q) + g;
    float q[D], acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        q[d] = qp[d];
        acc[d] = 0.f;
    }
    const float* kh = static_cast<const float*>(p.kreg) + static_cast<size_t>(h) * p.rows * D;
    const float* vh = static_cast<const float*>(p.vreg) + static_cast<size_t>(h) * D * p.rows;
    const float sl2 = p.scale_log2;
    float m = -INFINITY, l = 0.f;
    for (int sgi = 0; sgi < segs.n(); ++sgi) {
        const int lo = segs.lo(sgi);
        const int hi = segs.hi(sgi);
        for (int key = lo; key < hi; ++key) {
            const float* kp = kh + static_cast<size_t>(key) * D;
            float s = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) s = fmaf(q[d], kp[d], s);
            s *= sl2;
            const float mnew = fmaxf(m, s);
            const float alpha = exp2f(m - mnew);
            const float pr = exp2f(s - mnew);
            l = l * alpha + pr;
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] = fmaf(pr, vh[vt_elem(d, vt_pos(key), D)], acc[d] * alpha);
            m = mnew;
        }
    }
    float* op = static_cast<float*>(p.out) + g;
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
    if (p.lse != nullptr)
        p.lse[static_cast<size_t>(h) * p.nq * (PREFILL ? p.F : 1) + static_cast<size_t>(frame) * p.nq + r] =
            (m + log2f(l)) * 0.69314718055994530942f;
}

#ifndef SWA_NW
#define SWA_NW 4
#endif
#ifndef SWA_QB
#define SWA_QB 1
#endif
#ifndef SWA_OCC
#define SWA_OCC 3
#endif
constexpr int kNW = SWA_NW;       // waves per work-group
constexpr int kQB = SWA_QB;       // 32-query blocks per wave
constexpr int kOcc = SWA_OCC;     // waves per SIMD the register budget targets

template <int D, bool PRE>
void attn_bf16_launch(bool prefill, const AttnParams& p, int grid, hipStream_t stream) {
    if (!prefill && p.dseg != nullptr)
        hipLaunchKernelGGL((attn_bf16_kernel<D, kNW, kQB, kOcc, false, true, PRE>), dim3(grid), dim3(kNW * 64), 0,
                           stream, p);
    else if (prefill)
        hipLaunchKernelGGL((attn_bf16_kernel<D, kNW, kQB, kOcc, true, false, PRE>), dim3(grid), dim3(kNW * 64), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<D, kNW, kQB, kOcc, false, false, PRE>), dim3(grid), dim3(kNW * 64), 0,
                           stream, p);
}

template <int D>
hipError_t attn_bf16_dispatch(bool prefill, const AttnParams& p, int grid, hipStream_t stream) {
    if (p.lse == nullptr)
        attn_bf16_launch<D, true>(prefill, p, grid, stream);
    else
        attn_bf16_launch<D, false>(prefill, p, grid, stream);
    return hipGetLastError();
}

template <int D>
hipError_t attn_f32_dispatch(bool prefill, const AttnParams& p, hipStream_t stream) {
    dim3 grid((p.nq + 63) / 64, p.H, prefill ? p.F : 1);
    if (prefill)
        hipLaunchKernelGGL((attn_f32_kernel<D, true>), grid, dim3(64), 0, stream, p);
    else
        hipLaunchKernelGGL((attn_f32_kernel<D, false>), grid, dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

template <typename K>
int blocks_per_cu_of(K kernel, int threads) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0);
    return (e == hipSuccess && n > 0) ? n : 1;
}

// The fewer of the two softmax variants' resident work-groups (the
// automatic split sizes one launch round with it).
int attention_blocks_per_cu(int dtype, int D) {
    if (dtype != 0) return 1;
    if (D == 64)
        return std::min(blocks_per_cu_of(attn_bf16_kernel<64, kNW, kQB, kOcc, false, false, false>, kNW * 64),
                        blocks_per_cu_of(attn_bf16_kernel<64, kNW, kQB, kOcc, false, false, true>, kNW * 64));
    return std::min(blocks_per_cu_of(attn_bf16_kernel<32, kNW, kQB, kOcc, false, false, false>, kNW * 64),
                    blocks_per_cu_of(attn_bf16_kernel<32, kNW, kQB, kOcc, false, false, true>, kNW * 64));
}

int attention_q_tile(int dtype) { return dtype == 0 ? Shape<kNW, kQB>::QROWS : 64; }

// Token decode: one wave per work-group; its 32 query rows are the query
// heads of one (sequence, kv head) pair.
int attention_decode_q_rows() { return Shape<1, 1>::QROWS; }

int attention_decode_blocks_per_cu(int D) {
    return D == 64 ? blocks_per_cu_of(attn_bf16_kernel<64, 1, 1, kOcc, false, false, false>, 64)
                   : blocks_per_cu_of(attn_bf16_kernel<32, 1, 1, kOcc, false, false, false>, 64);
}

template <int D, bool PRE>
void decode_launch(const AttnParams& p, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_bf16_kernel<D, 1, 1, kOcc, false, false, PRE>), dim3(grid), dim3(64), 0, stream, p);
}

// Decode keeps Q exact: it is bound by HBM, not by the softmax's vector
// work, and the pre-scaled variant would need more registers than two waves
// per SIMD allow.
hipError_t launch_attention_decode(int D, const AttnParams& p, int grid, hipStream_t stream) {
    if (D == 64)
        decode_launch<64, false>(p, grid, stream);
    else
        decode_launch<32, false>(p, grid, stream);
    return hipGetLastError();
}

hipError_t launch_attention(int dtype, int D, bool prefill, const AttnParams& p, int grid,
                            hipStream_t stream) {
    if (dtype == 0) return D == 64 ? attn_bf16_dispatch<64>(prefill, p, grid, stream)
                                   : attn_bf16_dispatch<32>(prefill, p, grid, stream);
    return D == 64 ? attn_f32_dispatch<64>(prefill, p, stream) : attn_f32_dispatch<32>(prefill, p, stream);
}

hipError_t launch_merge(int D, int H, int nq, int n, int ncols, const float* part_o, const float* part_ml, void* out,
                        float* lse, int64_t rs, int64_t hs, const int* dn, hipStream_t stream) {
    if (nq <= 32) {
        const int64_t ipb = 256 / kDecodeLanes;
        const int64_t blocks = static_cast<int64_t>(H) * ((static_cast<int64_t>(nq) * (D / 4) + ipb - 1) / ipb);
        if (D == 64)
            hipLaunchKernelGGL((merge_decode_kernel<64>), dim3(blocks), dim3(256), 0, stream, part_o, part_ml,
                               static_cast<uint16_t*>(out), lse, H, nq, n, ncols, rs, hs, dn);
        else
            hipLaunchKernelGGL((merge_decode_kernel<32>), dim3(blocks), dim3(256), 0, stream, part_o, part_ml,
                               static_cast<uint16_t*>(out), lse, H, nq, n, ncols, rs, hs, dn);
        return hipGetLastError();
    }
    const int total = H * nq * (D / 4);
    const dim3 grid((total + 255) / 256);
    if (D == 64)
        hipLaunchKernelGGL((merge_kernel<64>), grid, dim3(256), 0, stream, part_o, part_ml,
                           static_cast<uint16_t*>(out), lse, H, nq, n, ncols, rs, hs, dn);
    else
        hipLaunchKernelGGL((merge_kernel<32>), grid, dim3(256), 0, stream, part_o, part_ml,
                           static_cast<uint16_t*>(out), lse, H, nq, n, ncols, rs, hs, dn);
    return hipGetLastError();
}

}  // namespace swa
