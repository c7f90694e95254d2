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
//  * Keys stream through LDS in tiles of 64 rows (double-buffered): K as
//    [64][D] and V^T as [D][64] (both padded against bank conflicts).
//  * S^T = K Q^T: the accumulator layout puts one query per lane column and
//    16 keys per lane, so a query's row max needs one cross-half exchange
//    and the row sum stays lane-local until the end.
//  * The exponentiated scores are converted to bf16 in registers and used
//    directly as the B operand of O^T = V^T P^T: the key order inside each
//    16-key step follows the accumulator layout, and the V^T reads from LDS
//    pick the same key order, so no data moves between lanes.
//  * Online softmax in the log2 domain (scores scaled by log2(e)/sqrt(D));
//    the O rescale is skipped when no lane's running max changed.
//  * Segment edges: a tile starts on an 8-row boundary; keys outside the
//    segment get score -inf and zeroed V^T in LDS.
#include <math.h>

#include "launch.hpp"

namespace swa {

namespace {

constexpr int KT = 64;            // keys per tile

template <int NW, int QB>
struct Shape {
    static constexpr int NT = NW * 64;
    static constexpr int QROWS = NW * QB * 32;
};

__device__ __forceinline__ int tiles_of(int lo, int hi) {
    const int b = lo & ~7;
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

// Segment accessors: streaming reads the list from kernel arguments,
// prefill from the scalars above.
template <bool PREFILL>
struct SegSrc {
    const AttnParams& p;
    PreSegs pre;
    __device__ int n() const { return PREFILL ? pre.n : p.seg.n; }
    __device__ int total() const { return PREFILL ? pre.total : p.seg.total_tiles; }
    __device__ int lo(int j) const { return PREFILL ? (j == 0 ? pre.lo0 : pre.lo1) : p.seg.lo[j]; }
    __device__ int hi(int j) const { return PREFILL ? (j == 0 ? pre.hi0 : pre.hi1) : p.seg.hi[j]; }
    __device__ int tile0(int j) const { return PREFILL ? (j == 0 ? 0 : pre.t1) : p.seg.tile0[j]; }
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
    c.base = (c.lo & ~7) + (t - s.tile0(c.seg)) * KT;
    return c;
}

template <class Src>
__device__ __forceinline__ void cursor_next(const Src& s, Cursor* c) {
    c->base += KT;
    if (c->base >= c->hi && c->seg + 1 < s.n()) {
        c->seg += 1;
        c->lo = s.lo(c->seg);
        c->hi = s.hi(c->seg);
        c->base = c->lo & ~7;
    }
}

// Keep-mask of a word holding the bf16 values of keys `key` (low half) and
// `key + 1` (high half): an element outside [lo, hi) is cleared.
__device__ __forceinline__ uint32_t keep_mask(int key, int lo, int hi) {
    const uint32_t m0 = (key >= lo && key < hi) ? 0x0000FFFFu : 0u;
    const uint32_t m1 = (key + 1 >= lo && key + 1 < hi) ? 0xFFFF0000u : 0u;
    return m0 | m1;
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

// Global loads of one 64-key tile: K rows [base, base+64) and the matching
// 64 columns of every V^T row, 16 bytes per load.
template <int D, int NT>
__device__ __forceinline__ void tile_gload(const uint16_t* kh, const uint16_t* vh, int rows, int base, int tid,
                                           u32x4 (&kr)[KT * D / 8 / NT], u32x4 (&vr)[D * KT / 8 / NT]) {
#pragma unroll
    for (int i = 0; i < KT * D / 8 / NT; ++i) {
        const int c = tid + i * NT;
        const int row = c / (D / 8);
        const int ch = c % (D / 8);
        kr[i] = *reinterpret_cast<const u32x4*>(kh + static_cast<size_t>(base + row) * D + ch * 8);
    }
#pragma unroll
    for (int i = 0; i < D * KT / 8 / NT; ++i) {
        const int c = tid + i * NT;
        const int d = c / (KT / 8);
        const int kc = c % (KT / 8);
        vr[i] = *reinterpret_cast<const u32x4*>(vh + static_cast<size_t>(d) * rows + base + kc * 8);
    }
}

// Stores of the prefetched tile into one LDS buffer; V^T elements of keys
// outside the segment are cleared (K rows there are masked by score).
template <int D, int NT, int KLD, int VLD>
__device__ __forceinline__ void tile_lstore(uint16_t* ks, uint16_t* vs, const Cursor& c, int tid,
                                            const u32x4 (&kr)[KT * D / 8 / NT], const u32x4 (&vr)[D * KT / 8 / NT]) {
    const bool edge = c.base < c.lo || c.base + KT > c.hi;
#pragma unroll
    for (int i = 0; i < KT * D / 8 / NT; ++i) {
        const int cc = tid + i * NT;
        const int row = cc / (D / 8);
        const int ch = cc % (D / 8);
        *reinterpret_cast<u32x4*>(ks + row * KLD + ch * 8) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < D * KT / 8 / NT; ++i) {
        const int cc = tid + i * NT;
        const int d = cc / (KT / 8);
        const int kc = cc % (KT / 8);
        u32x4 u = vr[i];
        if (edge) {
            const int k0 = c.base + kc * 8;
            u.x &= keep_mask(k0 + 0, c.lo, c.hi);
            u.y &= keep_mask(k0 + 2, c.lo, c.hi);
            u.z &= keep_mask(k0 + 4, c.lo, c.hi);
            u.w &= keep_mask(k0 + 6, c.lo, c.hi);
        }
        u32x2* dst = reinterpret_cast<u32x2*>(vs + d * VLD + kc * 8);
        dst[0] = u.xy;
        dst[1] = u.zw;
    }
}

template <int D, int NW, int QB, bool PREFILL>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(AttnParams p) {
    using Sh = Shape<NW, QB>;
    constexpr int NT = Sh::NT;
    constexpr int KLD = D + 8;                   // K tile row stride (elements)
    constexpr int VLD = KT + 4;                  // V^T tile row stride
    constexpr int CK = KT * D / 8 / NT;          // 16-byte K chunks per thread
    constexpr int CV = D * KT / 8 / NT;          // 16-byte V^T chunks per thread
    static_assert(CK * NT == KT * D / 8 && CV * NT == D * KT / 8, "tile/thread mismatch");
    constexpr int KS = D / 16;                   // MFMA k-steps of S^T = K Q^T
    constexpr int DB = D / 32;                   // 32-row feature blocks of O^T

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KLD];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][D * VLD];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hl = lane >> 5;                    // lane half

    // ---- work item ------------------------------------------------------------
    const int G = gridDim.x;
    const int L = xcd_remap(blockIdx.x, G);
    const int qt = L % p.qtiles;
    const int grp = L / p.qtiles;
    int h, split, frame;
    PreSegs pre{};
    if constexpr (PREFILL) {
        h = grp % p.H;
        frame = p.F - 1 - grp / p.H;             // heaviest frames first
        split = 0;
        pre = prefill_segs(frame, p.W, p.S, p.fP);
    } else {
        h = grp / p.splits;
        split = grp % p.splits;
        frame = 0;
    }
    const SegSrc<PREFILL> segs{p, pre};
    const int t_begin = static_cast<int>((static_cast<int64_t>(segs.total()) * split) / p.splits);
    const int t_end = static_cast<int>((static_cast<int64_t>(segs.total()) * (split + 1)) / p.splits);
    const int ntiles = t_end - t_begin;

    const uint16_t* kh = static_cast<const uint16_t*>(p.kreg) + static_cast<size_t>(h) * p.rows * D;
    const uint16_t* vh = static_cast<const uint16_t*>(p.vreg) + static_cast<size_t>(h) * D * p.rows;

    // ---- Q^T operands ----------------------------------------------------------
    const int qrow0 = qt * Sh::QROWS + wave * QB * 32;
    bf16x8 qf[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int r = qrow0 + qb * 32 + l32;
        const bool ok = r < p.nq;
        const size_t g = (static_cast<size_t>(frame) * p.nq + (ok ? r : 0)) * p.H + h;
        const uint16_t* src = static_cast<const uint16_t*>(p.q) + g * D + hl * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 u = ok ? *reinterpret_cast<const u32x4*>(src + ks * 16) : u32x4{0u, 0u, 0u, 0u};
            qf[qb][ks] = __builtin_bit_cast(bf16x8, u);
        }
    }

    f32x16 o[QB][DB];
    float m[QB], l[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        l[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[qb][db][i] = 0.f;
    }

    // ---- tile loader (registers -> LDS, double-buffered) -----------------------
    u32x4 kr[CK], vr[CV];
    const float sl2 = p.scale_log2;
    Cursor cur = cursor_at(segs, t_begin);
    if (ntiles > 0) {
        tile_gload<D, NT>(kh, vh, p.rows, cur.base, tid, kr, vr);
        tile_lstore<D, NT, KLD, VLD>(Ks[0], Vs[0], cur, tid, kr, vr);
    }
    Cursor nxt = cur;

    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        const bool more = it + 1 < ntiles;
        if (more) {
            cursor_next(segs, &nxt);
            tile_gload<D, NT>(kh, vh, p.rows, nxt.base, tid, kr, vr);
        }
        __syncthreads();

        // S^T = K Q^T for two 32-key blocks
        f32x16 s[2][QB];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][qb][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(&Ks[buf][(kb * 32 + l32) * KLD + ks * 16 + hl * 8]);
                const bf16x8 av = __builtin_bit_cast(bf16x8, a);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[qb][ks], s[kb][qb], 0, 0, 0);
            }
        }

        // keys outside the segment (only on its first and last tile)
        if (cur.base < cur.lo || cur.base + KT > cur.hi) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = cur.base + kb * 32 + 8 * (i >> 2) + 4 * hl + (i & 3);
                    if (key < cur.lo || key >= cur.hi) {
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) s[kb][qb][i] = -INFINITY;
                    }
                }
        }

        // online softmax (log2 domain) and P^T in bf16
        bf16x8 pb[2][QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = s[0][qb][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][qb][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m[qb], mx * sl2);
            const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
            if (__builtin_amdgcn_ballot_w64(mnew > m[qb]) != 0) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha;
                l[qb] *= alpha;
            }
            m[qb] = mnew;
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][hf * 8 + 2 * e], sl2, -mnew));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][hf * 8 + 2 * e + 1], sl2, -mnew));
                        ls += p0 + p1;
                        w[e] = pack_bf2(p0, p1);
                    }
                    pb[kb][qb][hf] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
                }
            l[qb] += ls;
        }

        // O^T += V^T P^T, 16 keys per step in the accumulator's key order
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint16_t* vp = &Vs[buf][(db * 32 + l32) * VLD + kb * 32 + hf * 16 + 4 * hl];
                    const u32x2 lo2 = *reinterpret_cast<const u32x2*>(vp);
                    const u32x2 hi2 = *reinterpret_cast<const u32x2*>(vp + 8);
                    const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{lo2.x, lo2.y, hi2.x, hi2.y});
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kb][qb][hf], o[qb][db], 0, 0, 0);
                }

        if (more) tile_lstore<D, NT, KLD, VLD>(Ks[buf ^ 1], Vs[buf ^ 1], nxt, tid, kr, vr);
        cur = nxt;
    }

    // ---- epilogue ------------------------------------------------------------------
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = l[qb] + __shfl_xor(l[qb], 32);
        const int r = qrow0 + qb * 32 + l32;
        if (r >= p.nq) continue;
        if (p.splits == 1) {
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            const size_t g = (static_cast<size_t>(frame) * p.nq + r) * p.H + h;
            uint16_t* dst = static_cast<uint16_t*>(p.out) + g * D;
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
            const size_t row = (static_cast<size_t>(split) * p.H + h) * p.nq + r;
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
    const size_t g = (static_cast<size_t>(frame) * p.nq + r) * p.H + h;
    const float* qp = static_cast<const float*>(p.q) + g * D;
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
            for (int d = 0; d < D; ++d) acc[d] = fmaf(pr, vh[static_cast<size_t>(d) * p.rows + key], acc[d] * alpha);
            m = mnew;
        }
    }
    float* op = static_cast<float*>(p.out) + g * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
    if (p.lse != nullptr)
        p.lse[static_cast<size_t>(h) * p.nq * (PREFILL ? p.F : 1) + static_cast<size_t>(frame) * p.nq + r] =
            (m + log2f(l)) * 0.69314718055994530942f;
}

// Merge split partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <typename TO, int D>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, TO* __restrict__ out,
                                                      float* __restrict__ lse, int H, int nq, int splits) {
    constexpr int C = D / 4;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= nq * H * C) return;
    const int chunk = idx % C;
    const int hq = idx / C;
    const int q = hq / H;
    const int h = hq % H;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s)
        M = fmaxf(M, part_ml[((static_cast<size_t>(s) * H + h) * nq + q) * 2]);
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < splits; ++s) {
        const size_t row = (static_cast<size_t>(s) * H + h) * nq + q;
        const float ms = part_ml[row * 2];
        const float w = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
        L += w * part_ml[row * 2 + 1];
        const float4 v = *reinterpret_cast<const float4*>(part_o + row * D + chunk * 4);
        acc.x += w * v.x;
        acc.y += w * v.y;
        acc.z += w * v.z;
        acc.w += w * v.w;
    }
    const float inv = 1.f / L;
    const size_t g = (static_cast<size_t>(q) * H + h) * D + chunk * 4;
    if constexpr (sizeof(TO) == 2) {
        const uint32_t w0 = pack_bf2(acc.x * inv, acc.y * inv);
        const uint32_t w1 = pack_bf2(acc.z * inv, acc.w * inv);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + g) = make_uint2(w0, w1);
    } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + g) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    if (lse != nullptr && chunk == 0) lse[static_cast<size_t>(h) * nq + q] = (M + log2f(L)) * 0.69314718055994530942f;
}

constexpr int kNW = 2;
constexpr int kQB = 2;

template <int D>
hipError_t attn_bf16_dispatch(bool prefill, const AttnParams& p, int grid, hipStream_t stream) {
    if (prefill)
        hipLaunchKernelGGL((attn_bf16_kernel<D, kNW, kQB, true>), dim3(grid), dim3(kNW * 64), 0, stream, p);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<D, kNW, kQB, false>), dim3(grid), dim3(kNW * 64), 0, stream, p);
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

int attention_q_tile(int dtype) { return dtype == 0 ? Shape<kNW, kQB>::QROWS : 64; }

hipError_t launch_attention(int dtype, int D, bool prefill, const AttnParams& p, int grid,
                            hipStream_t stream) {
    if (dtype == 0) return D == 64 ? attn_bf16_dispatch<64>(prefill, p, grid, stream)
                                   : attn_bf16_dispatch<32>(prefill, p, grid, stream);
    return D == 64 ? attn_f32_dispatch<64>(prefill, p, stream) : attn_f32_dispatch<32>(prefill, p, stream);
}

hipError_t launch_combine(int dtype, int D, int H, int nq, int splits, const float* part_o,
                          const float* part_ml, void* out, float* lse, hipStream_t stream) {
    const int n = nq * H * (D / 4);
    const dim3 grid((n + 255) / 256);
    if (dtype == 0) {
        if (D == 64)
            hipLaunchKernelGGL((combine_kernel<uint16_t, 64>), grid, dim3(256), 0, stream, part_o, part_ml,
                               static_cast<uint16_t*>(out), lse, H, nq, splits);
        else
            hipLaunchKernelGGL((combine_kernel<uint16_t, 32>), grid, dim3(256), 0, stream, part_o, part_ml,
                               static_cast<uint16_t*>(out), lse, H, nq, splits);
    } else {
        if (D == 64)
            hipLaunchKernelGGL((combine_kernel<float, 64>), grid, dim3(256), 0, stream, part_o, part_ml,
                               static_cast<float*>(out), lse, H, nq, splits);
        else
            hipLaunchKernelGGL((combine_kernel<float, 32>), grid, dim3(256), 0, stream, part_o, part_ml,
                               static_cast<float*>(out), lse, H, nq, splits);
    }
    return hipGetLastError();
}

}  // namespace swa
