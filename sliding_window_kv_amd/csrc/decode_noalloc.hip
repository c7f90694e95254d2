// Token decode that allocates nothing: the split partials live in a static
// device array instead of a caller workspace, for callers that cannot
// allocate device memory (stream capture, tight serving loops).
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.hpp"
#include "swa.h"

namespace {

// One copy per GPU, held until the process ends.  Host code must never pass
// `scratch` itself to a kernel: its device address comes from
// hipGetSymbolAddress, once per device with that device current.
constexpr size_t kScratchBytes = SWA_DECODE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (looked up on the first
// call on a device).
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return swa::api_fail(SWA_E_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return swa::api_fail(SWA_E_UNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) return swa::api_fail(SWA_E_HIP, "hipGetSymbolAddress of the decode scratch failed");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SWA_OK;
}

}  // namespace

extern "C" {

int swa_decode_step_noalloc(void* cache, size_t cache_bytes, int B, int Hq, int Hkv, int W, int D, int64_t pos,
                            const void* q, const void* k, const void* v, void* out, float* lse,
                            swa_stream_t stream) {
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || (D != 32 && D != 64))
        return swa::decode_step_impl(cache, cache_bytes, B, Hq, Hkv, W, D, pos, q, k, v, out, lse, nullptr, 1,
                                     stream);   // reports the argument error
    // the allocating entry point's split, so its partials must fit
    const int G = Hq / Hkv;
    if (swa::decode_partials_bytes(G, D, swa::kMaxDecodeCols) > static_cast<int64_t>(kScratchBytes))
        return swa::api_fail(SWA_E_CAPACITY,
                             "decode split partials exceed the 16 MiB static scratch: need "
                             "(Hq / Hkv) * (head_dim + 2) <= 1024");
    void* part = nullptr;
    const int rc = scratch_address(&part);
    if (rc != SWA_OK) return rc;
    return swa::decode_step_impl(cache, cache_bytes, B, Hq, Hkv, W, D, pos, q, k, v, out, lse, part,
                                 swa::kMaxDecodeCols, stream);
}

}  // extern "C"
