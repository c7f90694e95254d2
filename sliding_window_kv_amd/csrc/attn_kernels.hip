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
//  * Keys stream through LDS in tiles of 64 rows, double-buffered, loaded
//    with direct global->LDS 16-byte loads (no staging registers).  K is
//    kept as [64][D], V^T as [D][64]; 16-byte chunks are XOR-swizzled by row
//    so the MFMA operand reads are free of bank conflicts.
//  * S^T = K Q^T: the accumulator layout puts one query per lane column and
//    16 keys per lane, so a query's row max needs one cross-half exchange
//    and the row sum stays lane-local until the end.
//  * The exponentiated scores are converted to bf16 in registers and used
//    directly as the B operand of O^T = V^T P^T: the key order inside each
//    16-key step follows the accumulator layout, and V^T is stored with that
//    order (vt_pos), so each lane's A operand is one 16-byte LDS read.
//  * Online softmax in the log2 domain (scores scaled by log2(e)/sqrt(D));
//    the row sum is taken over the bf16 probabilities the MFMA consumes
//    (v_dot2), and the O rescale is skipped when no lane's running max
//    changed.
//  * Segment edges: tiles start on a 16-row boundary; keys outside the
//    segment get score -inf and their V^T elements are cleared in LDS.
#include <math.h>

#include "launch.hpp"

namespace swa {

namespace {

constexpr int KT = 64;            // keys per tile
constexpr int KALIGN = 16;        // tile start alignment (rows)

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

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Direct global->LDS loads of one tile (16 bytes per lane; a wave
// instruction fills 64 consecutive 16-byte LDS chunks).  LDS chunk p of the
// K buffer holds row p / CPR, feature chunk (p % CPR) ^ lds_swz(row); chunk
// p of the V^T buffer holds feature row p / 8, key chunk (p % 8) ^ lds_swz(row).
template <int D, int NW>
__device__ __forceinline__ void tile_load_lds(const uint16_t* kh, const uint16_t* vh, int rows, int base,
                                              uint16_t* ks, uint16_t* vs, int wave, int lane) {
    constexpr int CPR = D / 8;
    constexpr int NK = KT * CPR / (64 * NW);
    constexpr int NV = D * (KT / 8) / (64 * NW);
    static_assert(NK * 64 * NW == KT * CPR && NV * 64 * NW == D * (KT / 8), "tile/wave mismatch");
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int p0 = (i * NW + wave) * 64;
        const int p = p0 + lane;
        const int row = p / CPR;
        const int dc = (p % CPR) ^ lds_swz<CPR>(row);
        const uint16_t* g = kh + static_cast<size_t>(base + row) * D + dc * 8;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                         (__attribute__((address_space(3))) void*)(ks + p0 * 8), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int p0 = (i * NW + wave) * 64;
        const int p = p0 + lane;
        const int d = p / 8;
        const int kc = (p % 8) ^ lds_swz<8>(d);
        const uint16_t* g = vh + static_cast<size_t>(d) * rows + base + kc * 8;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                         (__attribute__((address_space(3))) void*)(vs + p0 * 8), 16, 0, 0);
    }
}

// Clear the V^T elements of keys outside [c.lo, c.hi) in a landed tile.
template <int D, int NT>
__device__ __forceinline__ void tile_clear_edges(uint16_t* vs, const Cursor& c, int tid) {
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

// ---------------------------------------------------------------------------
// Software-pipelined bf16 kernel (one wave per SIMD).  Iteration j runs the
// softmax of tile j on the vector ALUs while the matrix cores compute
// S_{j+1} = K_{j+1} Q^T and O += V_{j-1} P_{j-1}; the two streams are
// interleaved instruction by instruction with scheduling barriers.  K and
// V^T tiles are double-buffered and loaded one iteration ahead.
// ---------------------------------------------------------------------------

template <int D, int NW>
__device__ __forceinline__ void load_k_lds(const uint16_t* kh, int base, uint16_t* ks, int wave, int lane) {
    constexpr int CPR = D / 8;
    constexpr int NK = KT * CPR / (64 * NW);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        const int p0 = (i * NW + wave) * 64;
        const int p = p0 + lane;
        const int row = p / CPR;
        const int dc = (p % CPR) ^ lds_swz<CPR>(row);
        const uint16_t* g = kh + static_cast<size_t>(base + row) * D + dc * 8;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                         (__attribute__((address_space(3))) void*)(ks + p0 * 8), 16, 0, 0);
    }
}

template <int D, int NW>
__device__ __forceinline__ void load_v_lds(const uint16_t* vh, int rows, int base, uint16_t* vs, int wave, int lane) {
    constexpr int NV = D * (KT / 8) / (64 * NW);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int p0 = (i * NW + wave) * 64;
        const int p = p0 + lane;
        const int d = p / 8;
        const int kc = (p % 8) ^ lds_swz<8>(d);
        const uint16_t* g = vh + static_cast<size_t>(d) * rows + base + kc * 8;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                         (__attribute__((address_space(3))) void*)(vs + p0 * 8), 16, 0, 0);
    }
}

// Exchange between the two 32-lane halves of a wave: after the swap, `a`
// holds the lower half's values in both halves and `b` the upper half's, so
// max(a, b) and a + b combine each lane with lane ^ 32.  Written as inline
// assembly with both registers read-write: the compiler's builtin for this
// instruction returned the same register for both results.  The leading
// s_nop covers the VALU-write -> permlane-read hazard.
__device__ __forceinline__ void xhalf_swap(float x, float* lo, float* hi) {
    unsigned a = __builtin_bit_cast(unsigned, x);
    unsigned b = a;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
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

template <int D, int QB, bool DO_S, bool DO_PV>
__device__ __forceinline__ void pipe_step(f32x16 (&s)[2][QB], bf16x8 (&pcur)[2][QB][2], const bf16x8 (&pprev)[2][QB][2],
                                          f32x16 (&o)[QB][D / 32], float (&m)[QB], float (&l)[QB],
                                          const bf16x8 (&qf)[QB][D / 16], const uint16_t* kb_lds,
                                          const uint16_t* vb_lds, const Cursor& cs, float sl2, int l32, int hl) {
    constexpr int CPR = D / 8;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    static_assert(QB == 1 || QB == 2, "one or two query blocks per wave");
    constexpr int NB = 2 * QB;                   // 32x32 score blocks per tile
    constexpr int PPB = 4 / NB;                  // PV 16-key steps per block
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    const int ksw = lds_swz<CPR>(l32);
    const int vsw = lds_swz<8>(l32);

    // keys outside the segment get -inf (first/last tile of a segment only)
    if (cs.base < cs.lo || cs.base + KT > cs.hi) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = cs.base + kb * 32 + 8 * (i >> 2) + 4 * hl + (i & 3);
                if (key < cs.lo || key >= cs.hi) {
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[kb][qb][i] = -INFINITY;
                }
            }
    }

    // row max of tile j, running max, rescale factor
    float mnew[QB], alpha[QB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float mx = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][qb][i]);
        mx = xhalf_max(mx);
        mnew[qb] = fmaxf(m[qb], mx * sl2);
        alpha[qb] = __builtin_amdgcn_exp2f(m[qb] - mnew[qb]);
        need = need || (__builtin_amdgcn_ballot_w64(mnew[qb] > m[qb]) != 0);
        l[qb] *= alpha[qb];
        m[qb] = mnew[qb];
    }

    const f32x16 zero16 = {};
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int kb = b / QB;                   // block of tile j / S_{j+1}
        const int qb = b % QB;
        u32x4 ka[KS];
        if constexpr (DO_S) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int row = kb * 32 + l32;
                ka[ks] = *reinterpret_cast<const u32x4*>(kb_lds + (row * CPR + ((ks * 2 + hl) ^ ksw)) * 8);
            }
        }
        u32x4 va[PPB][DB];
        if constexpr (DO_PV) {
#pragma unroll
            for (int pp = 0; pp < PPB; ++pp) {
                const int pr = b * PPB + pp;     // PV step (kbv, hfv) = 16 keys of tile j-1
                const int kbv = pr / 2;
                const int hfv = pr % 2;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int d = db * 32 + l32;
                    const int kc = kbv * 4 + hfv * 2 + hl;
                    va[pp][db] = *reinterpret_cast<const u32x4*>(vb_lds + d * KT + ((kc ^ vsw) * 8));
                }
            }
        }
        // softmax of block (kb, qb) of tile j
        float ls = l[qb];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][hf * 8 + 2 * e], sl2, -mnew[qb]));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][hf * 8 + 2 * e + 1], sl2, -mnew[qb]));
                w[e] = pack_bf2(p0, p1);
                ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, ls, false);
            }
            pcur[kb][qb][hf] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
        }
        l[qb] = ls;
        // S_{j+1} for the same block, in the registers just consumed
        if constexpr (DO_S) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka[ks]), qf[qb][ks],
                                                                    ks == 0 ? zero16 : s[kb][qb], 0, 0, 0);
        }
        // this block's share of O += V_{j-1} P_{j-1}
        if constexpr (DO_PV) {
#pragma unroll
            for (int pp = 0; pp < PPB; ++pp) {
                const int pr = b * PPB + pp;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int q2 = 0; q2 < QB; ++q2)
                        o[q2][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, va[pp][db]), pprev[pr / 2][q2][pr % 2], o[q2][db], 0, 0, 0);
            }
        }
        constexpr int NM = (DO_S ? KS : 0) + (DO_PV ? PPB * DB * QB : 0);
        constexpr int ND = (DO_S ? KS : 0) + (DO_PV ? PPB * DB : 0);
        __builtin_amdgcn_sched_group_barrier(0x100, ND, 0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 48 / NM, 0);
        }
    }

    // O holds tiles up to j-1 relative to the previous max: bring it to m_j
    if (need) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha[qb];
    }
}

// Final O += V_{n-1} P_{n-1}.
template <int D, int QB>
__device__ __forceinline__ void pipe_last_pv(const bf16x8 (&pp)[2][QB][2], f32x16 (&o)[QB][D / 32],
                                             const uint16_t* vb_lds, int l32, int hl) {
    constexpr int DB = D / 32;
    const int vsw = lds_swz<8>(l32);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = db * 32 + l32;
                const int kc = kb * 4 + hf * 2 + hl;
                const u32x4 a = *reinterpret_cast<const u32x4*>(vb_lds + d * KT + ((kc ^ vsw) * 8));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pp[kb][qb][hf],
                                                                        o[qb][db], 0, 0, 0);
            }
}

// Final normalisation (split == 1) or the split partials (split > 1).
template <int D, int QB, bool PREFILL>
__device__ __forceinline__ void write_out(const AttnParams& p, const f32x16 (&o)[QB][D / 32], const float (&m)[QB],
                                          const float (&l)[QB], int qrow0, int frame, int h, int split, int l32,
                                          int hl) {
    constexpr int DB = D / 32;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = xhalf_sum(l[qb]);
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

// Per-lane element offsets of the 16-byte chunks a thread loads into one
// K tile ([64][D], swizzled) and one V^T tile ([D][64], swizzled); only the
// tile's first row changes from tile to tile, so every load is a uniform
// base plus one of these constant offsets.
template <int D, int NW>
struct TileOffsets {
    static constexpr int CPR = D / 8;
    static constexpr int NK = KT * CPR / (64 * NW);
    static constexpr int NV = D * (KT / 8) / (64 * NW);
    int k[NK];
    int v[NV];
    __device__ TileOffsets(int rows, int wave, int lane) {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int p = (i * NW + wave) * 64 + lane;
            const int row = p / CPR;
            k[i] = row * D + ((p % CPR) ^ lds_swz<CPR>(row)) * 8;
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int p = (i * NW + wave) * 64 + lane;
            const int d = p / 8;
            v[i] = d * rows + ((p % 8) ^ lds_swz<8>(d)) * 8;
        }
    }
};

// Direct global->LDS loads of the 64-key tile starting at row `base`.
template <int D, int NW>
__device__ __forceinline__ void tile_load(const TileOffsets<D, NW>& off, const uint16_t* kh, const uint16_t* vh,
                                          int base, uint16_t* ks, uint16_t* vs, int wave) {
    using TO = TileOffsets<D, NW>;
    const uint16_t* kt = kh + static_cast<size_t>(base) * D;
    const uint16_t* vt = vh + base;
#pragma unroll
    for (int i = 0; i < TO::NK; ++i)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kt + off.k[i]),
                                         (__attribute__((address_space(3))) void*)(ks + (i * NW + wave) * 512), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < TO::NV; ++i)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vt + off.v[i]),
                                         (__attribute__((address_space(3))) void*)(vs + (i * NW + wave) * 512), 16, 0, 0);
}

// One tile of the straightforward schedule: S^T = K Q^T, online softmax,
// O^T += V^T P^T, all from the landed buffers (ks, vs) of tile `cur`.
template <int D, int QB>
__device__ __forceinline__ void basic_tile(const uint16_t* ks, const uint16_t* vs, const Cursor& cur,
                                           const bf16x8 (&qf)[QB][D / 16], f32x16 (&o)[QB][D / 32], float (&m)[QB],
                                           float (&l)[QB], float sl2, int l32, int hl) {
    constexpr int CPR = D / 8;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    const int ksw = lds_swz<CPR>(l32);
    const int vsw = lds_swz<8>(l32);

    f32x16 s[2][QB];
    const f32x16 zero16 = {};
#pragma unroll
    for (int ks_ = 0; ks_ < KS; ++ks_) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int row = kb * 32 + l32;
            const u32x4 a = *reinterpret_cast<const u32x4*>(ks + (row * CPR + ((ks_ * 2 + hl) ^ ksw)) * 8);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[qb][ks_],
                                                                    ks_ == 0 ? zero16 : s[kb][qb], 0, 0, 0);
        }
    }
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
    bf16x8 pb[2][QB][2];
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
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = db * 32 + l32;
                const int kc = kb * 4 + hf * 2 + hl;
                const u32x4 a = *reinterpret_cast<const u32x4*>(vs + d * KT + ((kc ^ vsw) * 8));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb[kb][qb][hf],
                                                                        o[qb][db], 0, 0, 0);
            }
}

// One iteration of the straightforward kernel: wait for tile `it`, clear its
// edge keys, start the loads of the next tile into the other buffers, then
// compute.  Buffers are distinct LDS variables chosen at compile time, so
// the direct loads are known not to alias the reads of this tile.
template <int D, int NW, int QB, class Src>
__device__ __forceinline__ void basic_iter(int it, int ntiles, Cursor& cur, Cursor& nxt, const Src& segs,
                                           const TileOffsets<D, NW>& off, const uint16_t* kh, const uint16_t* vh,
                                           uint16_t* kcur, uint16_t* vcur, uint16_t* knext, uint16_t* vnext,
                                           const bf16x8 (&qf)[QB][D / 16], f32x16 (&o)[QB][D / 32], float (&m)[QB],
                                           float (&l)[QB], float sl2, int tid) {
    const int lane = tid & 63;
    const int wave = tid >> 6;
    __syncthreads();                             // tile `it` landed; tile it-1 fully consumed
    if (cur.base < cur.lo || cur.base + KT > cur.hi) {
        tile_clear_edges<D, NW * 64>(vcur, cur, tid);
        __syncthreads();
    }
    if (it + 1 < ntiles) {
        cursor_next(segs, &nxt);
        tile_load<D, NW>(off, kh, vh, nxt.base, knext, vnext, wave);
    }
    basic_tile<D, QB>(kcur, vcur, cur, qf, o, m, l, sl2, lane & 31, lane >> 5);
    cur = nxt;
}

template <int D, int NW, int QB, int OCC, bool PREFILL>
__global__ __launch_bounds__(NW * 64, OCC) void attn_bf16_kernel(AttnParams p) {
    using Sh = Shape<NW, QB>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;

    __shared__ __attribute__((aligned(16))) uint16_t K0[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t K1[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t V0[D * KT];
    __shared__ __attribute__((aligned(16))) uint16_t V1[D * KT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hl = lane >> 5;

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
    const TileOffsets<D, NW> off(p.rows, wave, lane);

    Cursor cur = cursor_at(segs, t_begin);
    Cursor nxt = cur;
    if (ntiles > 0) tile_load<D, NW>(off, kh, vh, cur.base, K0, V0, wave);

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
    const float sl2 = p.scale_log2;

    int it = 0;
    for (; it + 1 < ntiles; it += 2) {
        basic_iter<D, NW, QB>(it, ntiles, cur, nxt, segs, off, kh, vh, K0, V0, K1, V1, qf, o, m, l, sl2, tid);
        basic_iter<D, NW, QB>(it + 1, ntiles, cur, nxt, segs, off, kh, vh, K1, V1, K0, V0, qf, o, m, l, sl2, tid);
    }
    if (it < ntiles)
        basic_iter<D, NW, QB>(it, ntiles, cur, nxt, segs, off, kh, vh, K0, V0, K1, V1, qf, o, m, l, sl2, tid);

    write_out<D, QB, PREFILL>(p, o, m, l, qrow0, frame, h, split, l32, hl);
}


// One pipeline iteration j with static buffer roles: K_t lives in buffer
// t % 2 and V_t in buffer t % 2.  The iteration reads K_{j+1} (kr) and
// V_{j-1} (vr) and fills the other buffers (kw, vw) with K_{j+2} and V_j.
// Using distinct LDS variables per buffer lets the compiler see that the
// direct loads never alias the reads, so no wait is inserted between them.
template <int D, int NW, int QB, class Src>
__device__ __forceinline__ void pipe_iter(int j, int n, f32x16 (&sreg)[2][QB], bf16x8 (&pcur)[2][QB][2],
                                          const bf16x8 (&pprev)[2][QB][2], Cursor& cm1, Cursor& c0, Cursor& c1,
                                          Cursor& c2, const Src& segs, f32x16 (&o)[QB][D / 32], float (&m)[QB],
                                          float (&l)[QB], const bf16x8 (&qf)[QB][D / 16], const uint16_t* kr,
                                          uint16_t* vr, uint16_t* kw, uint16_t* vw, const uint16_t* kh,
                                          const uint16_t* vh, int rows, float sl2, int tid) {
    constexpr int NT = NW * 64;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hl = lane >> 5;
    __syncthreads();                                   // K_{j+1}, V_{j-1} landed; K_j, V_{j-2} consumed
    if (j > 0 && (cm1.base < cm1.lo || cm1.base + KT > cm1.hi)) {
        tile_clear_edges<D, NT>(vr, cm1, tid);
        __syncthreads();
    }
    // loads one iteration ahead (past the last tile: reload the last one)
    load_k_lds<D, NW>(kh, c2.base, kw, wave, lane);
    load_v_lds<D, NW>(vh, rows, c0.base, vw, wave, lane);
    pipe_step<D, QB, true, true>(sreg, pcur, pprev, o, m, l, qf, kr, vr, c0, sl2, l32, hl);
    cm1 = c0;
    c0 = c1;
    c1 = c2;
    if (j + 3 < n) cursor_next(segs, &c2);
}

template <int D, int NW, int QB, int OCC, bool PREFILL>
__global__ __launch_bounds__(NW * 64, OCC) void attn_bf16_pipe_kernel(AttnParams p) {
    using Sh = Shape<NW, QB>;
    constexpr int NT = Sh::NT;
    constexpr int CPR = D / 8;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;

    __shared__ __attribute__((aligned(16))) uint16_t K0[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t K1[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t V0[D * KT];
    __shared__ __attribute__((aligned(16))) uint16_t V1[D * KT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hl = lane >> 5;

    // ---- work item ------------------------------------------------------------
    const int G = gridDim.x;
    const int L = xcd_remap(blockIdx.x, G);
    const int qt = L % p.qtiles;
    const int grp = L / p.qtiles;
    int h, split, frame;
    PreSegs pre{};
    if constexpr (PREFILL) {
        h = grp % p.H;
        frame = p.F - 1 - grp / p.H;
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
    const int n = t_end - t_begin;

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
    const float sl2 = p.scale_log2;

    if (n > 0) {
        // cursors of tiles j-1, j, j+1, j+2 (clamped to the last tile)
        Cursor c0 = cursor_at(segs, t_begin);
        Cursor c1 = c0;
        if (n > 1) cursor_next(segs, &c1);
        Cursor c2 = c1;
        if (n > 2) cursor_next(segs, &c2);
        Cursor cm1 = c0;

        // prologue: K_0, K_1 in flight; V1 cleared (iteration 0 multiplies it by P = 0)
        load_k_lds<D, NW>(kh, c0.base, K0, wave, lane);
        load_k_lds<D, NW>(kh, c1.base, K1, wave, lane);
        for (int e = tid; e < D * KT / 8; e += NT) reinterpret_cast<u32x4*>(V1)[e] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();

        f32x16 sreg[2][QB];
        bf16x8 PA[2][QB][2], PB[2][QB][2];
        {
            const f32x16 zero16 = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int row = kb * 32 + l32;
                    const u32x4 a = *reinterpret_cast<const u32x4*>(&K0[(row * CPR + ((ks * 2 + hl) ^ lds_swz<CPR>(l32))) * 8]);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        sreg[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, a), qf[qb][ks], ks == 0 ? zero16 : sreg[kb][qb], 0, 0, 0);
                }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) PB[kb][qb][hf] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        }

        int j = 0;
        for (; j + 1 < n; j += 2) {
            pipe_iter<D, NW, QB>(j, n, sreg, PA, PB, cm1, c0, c1, c2, segs, o, m, l, qf, K1, V1, K0, V0, kh, vh,
                                 p.rows, sl2, tid);
            pipe_iter<D, NW, QB>(j + 1, n, sreg, PB, PA, cm1, c0, c1, c2, segs, o, m, l, qf, K0, V0, K1, V1, kh, vh,
                                 p.rows, sl2, tid);
        }
        if (j < n)     // n odd: one more even iteration
            pipe_iter<D, NW, QB>(j, n, sreg, PA, PB, cm1, c0, c1, c2, segs, o, m, l, qf, K1, V1, K0, V0, kh, vh,
                                 p.rows, sl2, tid);

        // last tile's PV: V_{n-1} is in buffer (n-1) % 2, P_{n-1} in PA if n-1 is even
        __syncthreads();
        uint16_t* vl = ((n - 1) & 1) ? V1 : V0;
        if (cm1.base < cm1.lo || cm1.base + KT > cm1.hi) {
            tile_clear_edges<D, NT>(vl, cm1, tid);
            __syncthreads();
        }
        if ((n - 1) & 1)
            pipe_last_pv<D, QB>(PB, o, vl, l32, hl);
        else
            pipe_last_pv<D, QB>(PA, o, vl, l32, hl);
    }
    write_out<D, QB, PREFILL>(p, o, m, l, qrow0, frame, h, split, l32, hl);
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
            for (int d = 0; d < D; ++d) acc[d] = fmaf(pr, vh[static_cast<size_t>(d) * p.rows + vt_pos(key)], acc[d] * alpha);
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

#ifndef SWA_NW
#define SWA_NW 4
#endif
#ifndef SWA_QB
#define SWA_QB 1
#endif
#ifndef SWA_OCC
#define SWA_OCC 2
#endif
constexpr int kNW = SWA_NW;       // waves per work-group
constexpr int kQB = SWA_QB;       // 32-query blocks per wave
constexpr int kOcc = SWA_OCC;     // waves per SIMD the register budget targets

#ifndef SWA_PIPE
#define SWA_PIPE 0
#endif

template <int D>
hipError_t attn_bf16_dispatch(bool prefill, const AttnParams& p, int grid, hipStream_t stream) {
    if (SWA_PIPE) {
        if (prefill)
            hipLaunchKernelGGL((attn_bf16_pipe_kernel<D, kNW, kQB, kOcc, true>), dim3(grid), dim3(kNW * 64), 0, stream, p);
        else
            hipLaunchKernelGGL((attn_bf16_pipe_kernel<D, kNW, kQB, kOcc, false>), dim3(grid), dim3(kNW * 64), 0, stream, p);
        return hipGetLastError();
    }
    if (prefill)
        hipLaunchKernelGGL((attn_bf16_kernel<D, kNW, kQB, kOcc, true>), dim3(grid), dim3(kNW * 64), 0, stream, p);
    else
        hipLaunchKernelGGL((attn_bf16_kernel<D, kNW, kQB, kOcc, false>), dim3(grid), dim3(kNW * 64), 0, stream, p);
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
