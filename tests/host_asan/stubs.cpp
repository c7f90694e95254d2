// Kernel-launch entry points for a host-only build of the C ABI (ring
// bookkeeping under AddressSanitizer/UBSan).  Only bookkeeping-only caches
// are driven there, so none of these is ever called; each fails loudly if
// it is.
#include <cstdio>
#include <cstdlib>

#include "launch.hpp"

namespace swa {
namespace {
[[noreturn]] void no_device(const char* what) {
    std::fprintf(stderr, "host-only build: %s called\n", what);
    std::abort();
}
}  // namespace

hipError_t launch_append(int, int, int, int, int, int, const void*, const void*, void*, void*, void*, const int32_t*,
                         const RopeArgs*, const NormArgs*, int32_t*, int32_t, const RetainArgs&, const StepPlan*,
                         hipStream_t) {
    no_device("launch_append");
}
hipError_t launch_plan_store(const StepPlan&, StepPlan*, hipStream_t) { no_device("launch_plan_store"); }
hipError_t launch_qknorm(int, int, int, int, void*, void*, const NormArgs&, hipStream_t) { no_device("launch_qknorm"); }
hipError_t launch_rope(int, int, int, int, void*, void*, const int32_t*, const RopeArgs&, hipStream_t) {
    no_device("launch_rope");
}
hipError_t launch_builder(const BuilderArgs&, hipStream_t) { no_device("launch_builder"); }
hipError_t launch_mask(int, int, int, int, int, uint8_t*, hipStream_t) { no_device("launch_mask"); }
hipError_t launch_attention(int, int, bool, const AttnParams&, int, hipStream_t) { no_device("launch_attention"); }
int attention_q_tile(int dtype) { return dtype == 0 ? 128 : 64; }
int attention_blocks_per_cu(int, int) { return 1; }
hipError_t launch_merge(int, int, int, int, int, const float*, const float*, void*, float*, int64_t, int64_t,
                        const int*, hipStream_t) {
    no_device("launch_merge");
}
hipError_t launch_attention_decode(int, const AttnParams&, int, hipStream_t) { no_device("launch_attention_decode"); }
int attention_decode_blocks_per_cu(int) { return 1; }
int attention_decode_q_rows() { return 32; }

}  // namespace swa
