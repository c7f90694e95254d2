// Internal interface between the C ABI's sources (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swa {

// Record an error message for swa_last_error(); returns code.
int api_fail(int code, const char* msg);

// Bytes of split-partial scratch a decode call with at most max_cols columns
// uses for G query heads per kv head (O partials, then their (m, l)).
int64_t decode_partials_bytes(int G, int D, int max_cols);

// One token-decode step (swa_decode_step's arguments) with its split
// partials in part (at least decode_partials_bytes(G, D, max_cols) bytes,
// 256-byte aligned) and the work split capped at max_cols columns.
int decode_step_impl(void* cache, size_t cache_bytes, int B, int Hq, int Hkv, int W, int D, int64_t pos,
                     const void* q, const void* k, const void* v, void* out, float* lse, void* part,
                     int max_cols, hipStream_t stream);

constexpr int kMaxDecodeCols = 2048;         // columns of one decode call (2 partial slots each)

}  // namespace swa
