// Shared device helpers for the gfx950 kernels: element types, bf16
// conversion, the prefill visibility ranges and kernel argument structs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxSegs = 8;      // row segments per streaming attention call
constexpr int kMaxCols = 256;    // columns of one streaming attention call (2 partial slots each)

// Storage position of a key inside the transposed V region: within every
// aligned group of 16 keys, bits 2 and 3 of the key index are swapped, so
// that the 8 keys one MFMA lane supplies to O^T = V^T P^T (keys 4h..4h+3
// and 8+4h..8+4h+3 of a 16-key step, h = lane half) are 8 consecutive
// elements.  The map is its own inverse.
__host__ __device__ __forceinline__ int vt_pos(int key) {
    return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// Element offset, inside one head's transposed V region, of feature d at
// storage position s (= vt_pos of the key): the region is a sequence of
// blocks of 64 positions, each block a [D][64] matrix, so the V^T of a
// 64-aligned key tile is one contiguous block.
__host__ __device__ __forceinline__ int vt_elem(int d, int s, int D) {
    return (s & ~63) * D + d * 64 + (s & 63);
}

__device__ __forceinline__ float bf2f(uint16_t b) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats to packed bf16 (lo in bits 0..15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2v));
}

// Visible key frames of query frame i in a masked prefill (guide, "Mask
// Generation in CausalAttention", with scale frames kept): the scale range
// A = [0, min(S, i+1)) and the window B = [max(0, i - W + 1), i + 1)
// (W < 0: no window).  When they touch, A covers both and B is empty.
__host__ __device__ __forceinline__ void prefill_ranges(int i, int W, int S, int* a0, int* a1,
                                                         int* b0, int* b1) {
    const int ws = (W < 0) ? 0 : ((i - W + 1) > 0 ? (i - W + 1) : 0);
    const int se = (S < i + 1) ? S : (i + 1);
    const bool merged = ws <= se;
    *a0 = 0;
    *a1 = merged ? i + 1 : se;
    *b0 = merged ? i + 1 : ws;
    *b1 = i + 1;
}

__host__ __device__ __forceinline__ bool prefill_visible(int i, int j, int W, int S) {
    int a0, a1, b0, b1;
    prefill_ranges(i, W, S, &a0, &a1, &b0, &b1);
    return (j >= a0 && j < a1) || (j >= b0 && j < b1);
}

// Row segments in the layer's row space, passed by value.
struct SegList {
    int n;
    int lo[kMaxSegs];
    int hi[kMaxSegs];
    int tile0[kMaxSegs];     // first tile index of the segment
    int total_tiles;
};

// Ring plan of one streaming step in device memory.  The kernels of a
// captured step read their destination rows, metadata entries and key
// segments from here, so that one captured graph serves every frame.
struct StepPlan {
    int32_t row0;            // append: first destination row (slot * P)
    int32_t append_meta;     // append: int32 index into the layer's metadata receiving the frame id
    int32_t frame;           // frame id of the appended frame
    int32_t retain;          // 1: copy the displaced frame's special rows before the append
    int32_t retain_src;      // first special row of the displaced frame
    int32_t retain_dst;      // first row of its entry in the special ring
    int32_t retain_meta;     // int32 index into the metadata receiving the displaced frame id
    int32_t victim_frame;
    SegList seg;             // visible key segments after the append (and eviction)
};

struct AttnParams {
    const void* q;           // [nq_total, H, D] NHD
    const void* kreg;        // [H][rows][D]
    const void* vreg;        // [H][D][rows]  (V transposed)
    void* out;               // [nq_total, H, D]
    float* lse;              // [H, nq_total] or null
    float* part_o;           // [pieces][nq][D] streaming partials
    float* part_ml;          // [pieces][nq][2] their running max (log2 domain) and sum
    int nq;                  // query rows per frame (P)
    int H;
    // element offset of (frame, row r, head h) in q and out:
    // (frame * nq + r) * rs + h * hs  (frame tensors: rs = H * D, hs = D)
    int64_t rs, hs;
    int rows;                // row length of the K/V regions
    int ncols;               // streaming: columns of the (head, key tile) space
    int qtiles;              // query tiles per frame
    float scale_log2;        // log2(e) / sqrt(D)
    // prefill only
    int F;
    int W;
    int S;
    int fP;                  // key rows per frame in the region
    SegList seg;             // streaming only
    const SegList* dseg;     // streaming: the segments in device memory instead of seg (captured steps)
    // token decode: the new token's key and value ([H][D] each), written
    // into row dslot of their buffer by the work-group that reads its tile
    const void* dk;
    const void* dv;
    int dslot;
};

}  // namespace swa
