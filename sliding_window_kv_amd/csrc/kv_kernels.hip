// Data-movement kernels of the frame cache on gfx950: append (with the 3-D
// RoPE fused in), special-row retention, standalone RoPE, the device
// page-list builder and the prefill mask export.
//
// Cache layout of one layer (rows = the layer's row space):
//   K   [H][rows][D]  -- a key row is D contiguous elements
//   V^T [H][rows/64][D][64] -- transposed in blocks of 64 keys, keys stored
//                        at vt_pos(key) (bits 2 and 3 swapped inside each
//                        16-key group), so a 64-aligned key tile's V^T is
//                        one contiguous block and the attention kernel reads
//                        the 8 keys one MFMA lane needs as one 16-byte load
// A frame in page slot s owns rows [s*P, (s+1)*P) (guide "KV Cache Eviction
// Strategy": whole frames enter and leave the cache).
#include "launch.hpp"

namespace swa {

namespace {

template <typename T>
struct Elt;
template <>
struct Elt<uint16_t> {
    static constexpr int kPer16B = 8;
    __device__ static float ld(uint16_t x) { return bf2f(x); }
    __device__ static uint16_t st(float f) { return f2bf(f); }
};
template <>
struct Elt<float> {
    static constexpr int kPer16B = 4;
    __device__ static float ld(float x) { return x; }
    __device__ static float st(float f) { return f; }
};

// One 16-byte chunk of elements.
template <typename T>
union Chunk {
    uint4 u;
    T e[Elt<T>::kPer16B];
};

// The token's three positions and the frequencies of pairs p0 .. p0+NP-1,
// all loaded before any of them is used (the sine/cosine code between uses
// would otherwise hold each next load back).
template <int NP>
struct RopeIn {
    int pos[3];
    double freq[NP];
    RopeIn() = default;
    __device__ RopeIn(const RopeArgs& r, const int32_t* pos3, int p0) {
#pragma unroll
        for (int b = 0; b < 3; ++b) pos[b] = pos3[b];
#pragma unroll
        for (int j = 0; j < NP; ++j) freq[j] = r.freq[p0 + j];
    }
};

// Angle of pair p (band chosen by p) in revolutions, reduced to [-1/2, 1/2]
// in double, then the hardware sine and cosine, which take their argument in
// revolutions (absolute error about 1.3e-7 on that range, measured against
// double precision; far under half a bf16 unit of the rotated values).
__device__ __forceinline__ void rope_cs(const RopeArgs& r, const int (&pos)[3], double freq, int p, float* c,
                                        float* s) {
    const int band = p < r.pairs_t ? 0 : (p < r.pairs_t + r.pairs_h ? 1 : 2);
    const double inv_twopi = 0.15915494309189533576888376337251;
    const double rev = static_cast<double>(band == 0 ? pos[0] : band == 1 ? pos[1] : pos[2]) * (freq * inv_twopi);
    const float red = static_cast<float>(rev - rint(rev));
    *s = __builtin_amdgcn_sinf(red);
    *c = __builtin_amdgcn_cosf(red);
}

// Rotate the E/2 pairs of one 16-byte chunk of k and one of q in place (the
// angles of the token computed once for both).
template <typename T>
__device__ __forceinline__ void rope_chunk2(T* x, T* y, const RopeArgs& r, const RopeIn<Elt<T>::kPer16B / 2>& in,
                                            int p0) {
    constexpr int E = Elt<T>::kPer16B;
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
        float c, s;
        rope_cs(r, in.pos, in.freq[j], p0 + j, &c, &s);
        const float a = Elt<T>::ld(x[2 * j]), b = Elt<T>::ld(x[2 * j + 1]);
        const float qa = Elt<T>::ld(y[2 * j]), qb = Elt<T>::ld(y[2 * j + 1]);
        x[2 * j] = Elt<T>::st(a * c - b * s);
        x[2 * j + 1] = Elt<T>::st(a * s + b * c);
        y[2 * j] = Elt<T>::st(qa * c - qb * s);
        y[2 * j + 1] = Elt<T>::st(qa * s + qb * c);
    }
}

// Rotate E/2 pairs of one chunk of k and one of q held as floats (the
// angles of a token computed once for both).
template <int E>
__device__ __forceinline__ void rope_pairs2(float* x, float* y, const RopeArgs& r, const RopeIn<E / 2>& in, int p0) {
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
        float c, s;
        rope_cs(r, in.pos, in.freq[j], p0 + j, &c, &s);
        const float a = x[2 * j], b = x[2 * j + 1];
        x[2 * j] = a * c - b * s;
        x[2 * j + 1] = a * s + b * c;
        const float qa = y[2 * j], qb = y[2 * j + 1];
        y[2 * j] = qa * c - qb * s;
        y[2 * j + 1] = qa * s + qb * c;
    }
}

// Layer norm of one (token, head) row over head_dim, the row held as CPR
// consecutive lanes of E floats each: mean, then the biased variance of the
// centred values, both reduced across the CPR lanes; then weight and bias
// (w, b point at this lane's E features).  Every lane of the wave takes
// part in the reductions.
template <int CPR, int E>
__device__ __forceinline__ void row_layer_norm(float (&x)[E], const float* w, const float* b, float eps) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) s += x[e];
#pragma unroll
    for (int off = 1; off < CPR; off <<= 1) s += __shfl_xor(s, off);
    const float mean = s * (1.f / (CPR * E));
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        x[e] -= mean;
        ss = fmaf(x[e], x[e], ss);
    }
#pragma unroll
    for (int off = 1; off < CPR; off <<= 1) ss += __shfl_xor(ss, off);
    const float inv = 1.f / sqrtf(ss * (1.f / (CPR * E)) + eps);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = fmaf(x[e] * inv, w[e], b[e]);
}

// Threads of an append block of TR rows: one per 16-byte chunk of the
// block's rows, so that every thread has a single chunk of k, v (and q) to
// move and rotate.
template <typename T, int D, int TR>
constexpr int append_threads() { return TR * D / Elt<T>::kPer16B; }

// One block = TR destination rows (TR-aligned, TR = 32 or 64: half of or one
// whole V^T block) of one head.  A per-frame pass is bound by latency, and
// 32-row blocks, with twice as many work-groups in flight, measured faster
// there (16-row ones slower); a pass over many frames (the prefill's chunk
// layout) has work-groups to spare and runs faster with 64-row blocks.
template <typename T, int D, bool ROPE, bool NORM, int TR>
__global__ __launch_bounds__((append_threads<T, D, TR>())) void append_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                     T* __restrict__ kreg, T* __restrict__ vreg,
                                                     T* __restrict__ q, const int32_t* __restrict__ pos,
                                                     RopeArgs rope, NormArgs norm, int H, int n_tok, int row0,
                                                     int rows, int32_t* meta_slot, int32_t frame_id,
                                                     RetainArgs ret, const StepPlan* __restrict__ plan) {
    constexpr int E = Elt<T>::kPer16B;
    if (plan != nullptr) {                   // captured step: destination, ids and retention from the device plan
        row0 = plan->row0;
        if (ret.ns > 0 && plan->retain != 0) {
            ret.src_row = plan->retain_src;
            ret.dst_row = plan->retain_dst;
            ret.meta = meta_slot + plan->retain_meta;
            ret.frame = plan->victim_frame;
        } else {
            ret.ns = 0;
        }
        meta_slot += plan->append_meta;
        frame_id = plan->frame;
    }
    constexpr int CPR = D / E;               // 16-byte chunks per row
    constexpr int NT = append_threads<T, D, TR>();
    constexpr int kTileRows = TR;
    constexpr int LD = D + 2;                // padded LDS row
    __shared__ T vt[kTileRows * LD];

    const int h = blockIdx.y;
    const int base = (row0 & ~(kTileRows - 1)) + blockIdx.x * kTileRows;  // first destination row
    const int tid = threadIdx.x;

    if (meta_slot != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *meta_slot = frame_id;

    // Retention of the previous occupant's special rows: the block whose
    // rows hold some of them copies those (K rows, and their V^T columns,
    // whose positions vt_pos keeps inside the same 16-row group) to the
    // special ring, and only then overwrites them.
    {
        const int lo = ret.src_row > base ? ret.src_row : base;
        const int hi = ret.src_row + ret.ns < base + kTileRows ? ret.src_row + ret.ns : base + kTileRows;
        if (lo < hi) {                       // uniform over the block
            if (ret.meta != nullptr && lo == ret.src_row && h == 0 && tid == 0) *ret.meta = ret.frame;
            const int nr = hi - lo;
            const int shift = ret.dst_row - ret.src_row;
            T* kh = kreg + static_cast<size_t>(h) * rows * D;
            for (int i = tid; i < nr * D; i += NT) {
                const int r = lo + i / D;
                kh[static_cast<size_t>(r + shift) * D + i % D] = kh[static_cast<size_t>(r) * D + i % D];
            }
            T* vh = vreg + static_cast<size_t>(h) * D * rows;
            for (int i = tid; i < nr * D; i += NT) {
                const int d = i / nr;
                const int r = lo + i % nr;
                vh[vt_elem(d, vt_pos(r + shift), D)] = vh[vt_elem(d, vt_pos(r), D)];
            }
            __syncthreads();                 // every old row read before any is overwritten
        }
    }

    // Every thread's loads first, all in flight together; rows outside the
    // frame read token 0 and store nothing (every lane also takes part in
    // the norm's row reductions).
    constexpr int NC = kTileRows * CPR / NT;
    static_assert(NC * NT == kTileRows * CPR, "whole 16-byte chunks per thread");
    Chunk<T> kv[NC], vv[NC], qv[NC];
    RopeIn<E / 2> rin[ROPE ? NC : 1];
#pragma unroll
    for (int it = 0; it < NC; ++it) {
        const int c = tid + it * NT;
        const int tok = base + c / CPR - row0;
        const int t = (tok >= 0 && tok < n_tok) ? tok : 0;
        const size_t src = (static_cast<size_t>(t) * H + h) * D + (c % CPR) * E;
        kv[it].u = *reinterpret_cast<const uint4*>(k + src);
        vv[it].u = *reinterpret_cast<const uint4*>(v + src);
        if constexpr (NORM || ROPE) qv[it].u = *reinterpret_cast<const uint4*>(q + src);
        if constexpr (ROPE) rin[it] = RopeIn<E / 2>(rope, pos + 3 * t, (c % CPR) * E / 2);
    }
    // consumed here, so that no load is sunk into the conditional stores below
    // (it would then wait for the one before it)
#pragma unroll
    for (int it = 0; it < NC; ++it) {
        asm volatile("" ::"v"(kv[it].u.x), "v"(kv[it].u.y), "v"(kv[it].u.z), "v"(kv[it].u.w));
        asm volatile("" ::"v"(vv[it].u.x), "v"(vv[it].u.y), "v"(vv[it].u.z), "v"(vv[it].u.w));
        if constexpr (NORM || ROPE)
            asm volatile("" ::"v"(qv[it].u.x), "v"(qv[it].u.y), "v"(qv[it].u.z), "v"(qv[it].u.w));
        if constexpr (ROPE) {
            asm volatile("" ::"v"(rin[it].pos[0]), "v"(rin[it].pos[1]), "v"(rin[it].pos[2]));
#pragma unroll
            for (int j = 0; j < E / 2; ++j) asm volatile("" ::"v"(rin[it].freq[j]));
        }
    }
#pragma unroll
    for (int it = 0; it < NC; ++it) {
        const int c = tid + it * NT;
        const int rr = c / CPR;
        const int ch = c % CPR;
        const int r = base + rr;
        const int tok = r - row0;
        const bool ok = tok >= 0 && tok < n_tok;
        const int t = ok ? tok : 0;
        const size_t src = (static_cast<size_t>(t) * H + h) * D + ch * E;
        if constexpr (NORM) {
            float kf[E], qf[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                kf[e] = Elt<T>::ld(kv[it].e[e]);
                qf[e] = Elt<T>::ld(qv[it].e[e]);
            }
            row_layer_norm<CPR, E>(qf, norm.w + ch * E, norm.w + D + ch * E, norm.eps);
            row_layer_norm<CPR, E>(kf, norm.w + 2 * D + ch * E, norm.w + 3 * D + ch * E, norm.eps);
            if constexpr (ROPE) rope_pairs2<E>(kf, qf, rope, rin[it], ch * E / 2);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                kv[it].e[e] = Elt<T>::st(kf[e]);
                qv[it].e[e] = Elt<T>::st(qf[e]);
            }
        } else if constexpr (ROPE) {
            rope_chunk2<T>(kv[it].e, qv[it].e, rope, rin[it], ch * E / 2);
        }
        if (ok) {
            if constexpr (NORM || ROPE) *reinterpret_cast<uint4*>(q + src) = qv[it].u;
            *reinterpret_cast<uint4*>(kreg + (static_cast<size_t>(h) * rows + r) * D + ch * E) = kv[it].u;
        } else {
            vv[it].u = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < E; ++e) vt[rr * LD + ch * E + e] = vv[it].e[e];
    }
    __syncthreads();

    // Transposed V, keys in vt_pos order: storage chunk kc of a feature row
    // holds the keys vt_pos(kc*E .. kc*E+E-1) of the tile, one 16-byte store
    // when all of them belong to the frame.
    constexpr int KC = kTileRows / E;        // storage chunks per feature
    for (int c = tid; c < D * KC; c += NT) {
        const int d = c / KC;
        const int kc = c % KC;
        Chunk<T> out;
        bool full = true;
        bool valid[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int key = vt_pos(kc * E + e);
            const int tok = base + key - row0;
            valid[e] = tok >= 0 && tok < n_tok;
            full = full && valid[e];
            out.e[e] = vt[key * LD + d];
        }
        T* dst = vreg + static_cast<size_t>(h) * D * rows + vt_elem(d, base + kc * E, D);
        if (full) {
            *reinterpret_cast<uint4*>(dst) = out.u;
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (valid[e]) dst[e] = out.e[e];
        }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kernel(T* __restrict__ q, T* __restrict__ k,
                                                   const int32_t* __restrict__ pos, RopeArgs rope,
                                                   int H, int n_tok) {
    constexpr int E = Elt<T>::kPer16B;
    constexpr int CPR = D / E;
    const int64_t n = static_cast<int64_t>(n_tok) * H * CPR;
    for (int64_t c = blockIdx.x * 256ll + threadIdx.x; c < n; c += static_cast<int64_t>(gridDim.x) * 256) {
        const int ch = static_cast<int>(c % CPR);
        const int tok = static_cast<int>(c / (CPR * H));
        // both loads before any use, so they are in flight together (a
        // missing tensor is rotated as garbage and not stored)
        Chunk<T> xq, xk;
        if (q != nullptr) xq.u = *reinterpret_cast<const uint4*>(q + c * E);
        if (k != nullptr) xk.u = *reinterpret_cast<const uint4*>(k + c * E);
        const RopeIn<E / 2> in(rope, pos + 3 * tok, ch * E / 2);
        rope_chunk2<T>(xk.e, xq.e, rope, in, ch * E / 2);
        if (q != nullptr) *reinterpret_cast<uint4*>(q + c * E) = xq.u;
        if (k != nullptr) *reinterpret_cast<uint4*>(k + c * E) = xk.u;
    }
}

// Per-head layer norm of q and k in place (either may be null); one thread
// per 16-byte chunk, the CPR chunks of a row in consecutive lanes.
template <typename T, int D>
__global__ __launch_bounds__(256) void qknorm_kernel(T* __restrict__ q, T* __restrict__ k, NormArgs norm, int64_t n) {
    constexpr int E = Elt<T>::kPer16B;
    constexpr int CPR = D / E;
    // grid-stride over whole waves, so the lanes of a row stay together and
    // every lane reaches the reductions (chunks past n compute on chunk 0)
    for (int64_t c0 = blockIdx.x * 256ll; c0 < n; c0 += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t c = c0 + threadIdx.x;
        const bool ok = c < n;
        const int64_t cc = ok ? c : 0;
        const int ch = static_cast<int>(cc % CPR);
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            T* x = which == 0 ? q : k;
            if (x == nullptr) continue;              // uniform
            Chunk<T> xv;
            xv.u = *reinterpret_cast<const uint4*>(x + cc * E);
            float f[E];
#pragma unroll
            for (int e = 0; e < E; ++e) f[e] = Elt<T>::ld(xv.e[e]);
            row_layer_norm<CPR, E>(f, norm.w + 2 * which * D + ch * E, norm.w + (2 * which + 1) * D + ch * E, norm.eps);
#pragma unroll
            for (int e = 0; e < E; ++e) xv.e[e] = Elt<T>::st(f[e]);
            if (ok) *reinterpret_cast<uint4*>(x + cc * E) = xv.u;
        }
    }
}

// Visible-page list from the device frame tables and the ring counters:
// scale frames, retained special entries (oldest first), window frames,
// pending non-keyframe.
__global__ __launch_bounds__(256) void builder_kernel(BuilderArgs a) {
    const int sc = a.W < 0 ? static_cast<int>(a.n_key) : static_cast<int>(min<int64_t>(a.n_key, a.S));
    const int64_t e0 = a.cross ? max<int64_t>(0, a.n_special - a.R) : 0;
    const int nsp = a.cross ? static_cast<int>(a.n_special - e0) : 0;
    for (int idx = threadIdx.x; idx < a.total; idx += blockDim.x) {
        int32_t frame, region, slot, row0, nrows;
        if (idx < sc) {
            frame = a.ord_frame[idx];
            region = 0;
            slot = idx;
            row0 = 0;
            nrows = a.P;
        } else if (idx < sc + nsp) {
            const int64_t e = e0 + (idx - sc);
            frame = a.special_frame[e % (a.R + 1)];
            region = 1;
            slot = static_cast<int>(e % a.R);
            row0 = slot * a.ns;
            nrows = a.ns;
        } else if (idx < sc + nsp + a.n_win) {
            const int64_t o = a.n_key - a.n_win + (idx - sc - nsp);
            frame = a.ord_frame[a.S + (o - a.S) % (a.W + 1)];
            region = 0;
            slot = a.S + static_cast<int>((o - a.S) % a.W);
            row0 = 0;
            nrows = a.P;
        } else {
            frame = *a.pending_frame;
            region = 0;
            slot = a.num_slots - 1;
            row0 = 0;
            nrows = a.P;
        }
        int32_t* o5 = a.out + 5 * idx;
        o5[0] = frame;
        o5[1] = region;
        o5[2] = slot;
        o5[3] = row0;
        o5[4] = nrows;
    }
}

__global__ __launch_bounds__(256) void mask_kernel(int F, int P, int W, int S, int token_level,
                                                   uint8_t* out) {
    const int64_t n = token_level ? static_cast<int64_t>(F) * P : F;
    const int64_t total = n * n;
    for (int64_t x = blockIdx.x * 256ll + threadIdx.x; x < total; x += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t r = x / n;
        const int64_t c = x % n;
        const int i = static_cast<int>(token_level ? r / P : r);
        const int j = static_cast<int>(token_level ? c / P : c);
        out[x] = prefill_visible(i, j, W, S) ? 1 : 0;
    }
}

template <typename T, int D, int kTileRows>
hipError_t append_dispatch(int H, int n_tok, int row0, int rows, const void* k, const void* v,
                           void* kreg, void* vreg, void* q, const int32_t* pos, const RopeArgs* rope,
                           const NormArgs* norm, int32_t* meta_slot, int32_t frame_id, const RetainArgs& ret,
                           const StepPlan* plan, hipStream_t stream) {
    const int first = row0 & ~(kTileRows - 1);
    // with a device plan the first row is not known here: enough tiles for any row offset
    const int tiles = plan != nullptr ? (kTileRows - 1 + n_tok + kTileRows - 1) / kTileRows
                                      : (row0 + n_tok - first + kTileRows - 1) / kTileRows;
    dim3 grid(tiles, H);
    RopeArgs r{};
    if (rope != nullptr) r = *rope;
    NormArgs nm{};
    if (norm != nullptr) nm = *norm;
#define SWA_APPEND(RO, NO)                                                                                  \
    hipLaunchKernelGGL((append_kernel<T, D, RO, NO, kTileRows>), grid, dim3(append_threads<T, D, kTileRows>()), \
                       0, stream,                                                                         \
                       static_cast<const T*>(k),                                                          \
                       static_cast<const T*>(v), static_cast<T*>(kreg), static_cast<T*>(vreg), static_cast<T*>(q), \
                       pos, r, nm, H, n_tok, row0, rows, meta_slot, frame_id, ret, plan)
    if constexpr (kTileRows == 64) {
        SWA_APPEND(false, false);
    } else {
        if (rope != nullptr && norm != nullptr)
            SWA_APPEND(true, true);
        else if (rope != nullptr)
            SWA_APPEND(true, false);
        else if (norm != nullptr)
            SWA_APPEND(false, true);
        else
            SWA_APPEND(false, false);
    }
#undef SWA_APPEND
    return hipGetLastError();
}

// 64-row blocks for plain (no RoPE, no norm) passes with at least 16
// work-groups of 32 rows per CU's worth (4096 of them), 32-row blocks
// otherwise.
template <typename T, int D>
hipError_t append_dispatch_any(int H, int n_tok, int row0, int rows, const void* k, const void* v, void* kreg,
                               void* vreg, void* q, const int32_t* pos, const RopeArgs* rope, const NormArgs* norm,
                               int32_t* meta_slot, int32_t frame_id, const RetainArgs& ret, const StepPlan* plan,
                               hipStream_t stream) {
    const bool big = rope == nullptr && norm == nullptr && (static_cast<int64_t>(n_tok) / 32) * H >= 4096;
    if (big)
        return append_dispatch<T, D, 64>(H, n_tok, row0, rows, k, v, kreg, vreg, q, pos, rope, norm, meta_slot,
                                         frame_id, ret, plan, stream);
    return append_dispatch<T, D, 32>(H, n_tok, row0, rows, k, v, kreg, vreg, q, pos, rope, norm, meta_slot,
                                     frame_id, ret, plan, stream);
}

}  // namespace

hipError_t launch_append(int dtype, int H, int D, int n_tok, int row0, int rows, const void* k,
                         const void* v, void* kreg, void* vreg, void* q, const int32_t* pos,
                         const RopeArgs* rope, const NormArgs* norm, int32_t* meta_slot, int32_t frame_id,
                         const RetainArgs& ret, const StepPlan* plan, hipStream_t stream) {
    if (dtype == 0) {
        if (D == 64)
            return append_dispatch_any<uint16_t, 64>(H, n_tok, row0, rows, k, v, kreg, vreg, q, pos, rope, norm,
                                                 meta_slot, frame_id, ret, plan, stream);
        return append_dispatch_any<uint16_t, 32>(H, n_tok, row0, rows, k, v, kreg, vreg, q, pos, rope, norm,
                                             meta_slot, frame_id, ret, plan, stream);
    }
    if (D == 64)
        return append_dispatch_any<float, 64>(H, n_tok, row0, rows, k, v, kreg, vreg, q, pos, rope, norm, meta_slot,
                                          frame_id, ret, plan, stream);
    return append_dispatch_any<float, 32>(H, n_tok, row0, rows, k, v, kreg, vreg, q, pos, rope, norm, meta_slot,
                                      frame_id, ret, plan, stream);
}

namespace {

// One streaming step's ring plan into device memory (arguments by value, so
// a later step's plan cannot overwrite this one before the launch).
__global__ __launch_bounds__(64) void plan_store_kernel(StepPlan plan, StepPlan* __restrict__ dst) {
    constexpr int N = static_cast<int>(sizeof(StepPlan) / 4);
    static_assert(N <= 64, "one wave stores the plan");
    const int i = threadIdx.x;
    if (i < N) reinterpret_cast<int32_t*>(dst)[i] = reinterpret_cast<const int32_t*>(&plan)[i];
}

}  // namespace

hipError_t launch_plan_store(const StepPlan& plan, StepPlan* dst, hipStream_t stream) {
    hipLaunchKernelGGL(plan_store_kernel, dim3(1), dim3(64), 0, stream, plan, dst);
    return hipGetLastError();
}

hipError_t launch_qknorm(int dtype, int n_tok, int H, int D, void* q, void* k, const NormArgs& norm,
                         hipStream_t stream) {
    const int64_t n = static_cast<int64_t>(n_tok) * H * D / (dtype == 0 ? 8 : 4);
    const int64_t want = (n + 255) / 256;
    const int blocks = static_cast<int>(want < 4096 ? want : 4096);
    if (dtype == 0) {
        if (D == 64)
            hipLaunchKernelGGL((qknorm_kernel<uint16_t, 64>), dim3(blocks), dim3(256), 0, stream,
                               static_cast<uint16_t*>(q), static_cast<uint16_t*>(k), norm, n);
        else
            hipLaunchKernelGGL((qknorm_kernel<uint16_t, 32>), dim3(blocks), dim3(256), 0, stream,
                               static_cast<uint16_t*>(q), static_cast<uint16_t*>(k), norm, n);
    } else {
        if (D == 64)
            hipLaunchKernelGGL((qknorm_kernel<float, 64>), dim3(blocks), dim3(256), 0, stream,
                               static_cast<float*>(q), static_cast<float*>(k), norm, n);
        else
            hipLaunchKernelGGL((qknorm_kernel<float, 32>), dim3(blocks), dim3(256), 0, stream,
                               static_cast<float*>(q), static_cast<float*>(k), norm, n);
    }
    return hipGetLastError();
}

hipError_t launch_rope(int dtype, int n_tok, int H, int D, void* q, void* k, const int32_t* pos,
                       const RopeArgs& rope, hipStream_t stream) {
    const int E = dtype == 0 ? 8 : 4;
    const int64_t chunks = static_cast<int64_t>(n_tok) * H * (D / E);
    int blocks = static_cast<int>((chunks + 255) / 256);
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    if (dtype == 0) {
        if (D == 64)
            hipLaunchKernelGGL((rope_kernel<uint16_t, 64>), dim3(blocks), dim3(256), 0, stream,
                               static_cast<uint16_t*>(q), static_cast<uint16_t*>(k), pos, rope, H, n_tok);
        else
            hipLaunchKernelGGL((rope_kernel<uint16_t, 32>), dim3(blocks), dim3(256), 0, stream,
                               static_cast<uint16_t*>(q), static_cast<uint16_t*>(k), pos, rope, H, n_tok);
    } else {
        if (D == 64)
            hipLaunchKernelGGL((rope_kernel<float, 64>), dim3(blocks), dim3(256), 0, stream,
                               static_cast<float*>(q), static_cast<float*>(k), pos, rope, H, n_tok);
        else
            hipLaunchKernelGGL((rope_kernel<float, 32>), dim3(blocks), dim3(256), 0, stream,
                               static_cast<float*>(q), static_cast<float*>(k), pos, rope, H, n_tok);
    }
    return hipGetLastError();
}

hipError_t launch_builder(const BuilderArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(builder_kernel, dim3(1), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_mask(int F, int P, int W, int S, int token_level, uint8_t* out,
                       hipStream_t stream) {
    const int64_t n = token_level ? static_cast<int64_t>(F) * P : F;
    int64_t blocks = (n * n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(mask_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, F, P, W,
                       S, token_level, out);
    return hipGetLastError();
}

}  // namespace swa
