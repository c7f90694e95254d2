// Host-side launchers of the gfx950 kernels (defined in the .hip files).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels_common.hpp"

namespace swa {

// 3-D RoPE band description (host-computed frequency ladder).
struct RopeArgs {
    int pairs_t, pairs_h, pairs_w;
    double freq[64];         // per pair: theta^(-kk / d_band)
};

// Per-head layer norm parameters: w = device float [4][D] (q weight, q bias,
// k weight, k bias).
struct NormArgs {
    const float* w;
    float eps;
};

// Special-row retention fused into an append: before the frame overwrites
// its slot, the ns rows starting at src_row of every head (K and V^T) are
// copied to dst_row, and meta, if not null, receives frame.  ns = 0: no copy.
// With a device plan (captured steps) the copy happens only if plan->retain,
// with rows, id and metadata entry (meta + plan->retain_meta) from the plan.
struct RetainArgs {
    int src_row, dst_row, ns;
    int32_t* meta;
    int32_t frame;
};

// Copy n_tok tokens of k, v ([n_tok, H, D]) into rows [row0, row0 + n_tok)
// of the K region ([H][rows][D]) and the transposed V region ([H][D][rows]).
// With norm != null, k is layer-normed per head on the way and q
// ([n_tok, H, D]) in place; with rope != null, k is rotated on the way and q
// in place (after the norm).  meta_slot, if not null, receives frame_id.
// With plan != null (captured steps) row0, frame_id and the metadata entry
// (meta_slot + plan->append_meta) are read from the device plan instead.
// `ret` is the retention of the special rows of the slot's previous
// occupant, done by the same launch before its rows are overwritten.
hipError_t launch_append(int dtype, int H, int D, int n_tok, int row0, int rows, const void* k,
                         const void* v, void* kreg, void* vreg, void* q, const int32_t* pos,
                         const RopeArgs* rope, const NormArgs* norm, int32_t* meta_slot, int32_t frame_id,
                         const RetainArgs& ret, const StepPlan* plan, hipStream_t stream);

// Store one step's ring plan into device memory (read by the kernels of a
// captured step).
hipError_t launch_plan_store(const StepPlan& plan, StepPlan* dst, hipStream_t stream);

// Per-head layer norm of q and/or k ([n_tok, H, D]) in place.
hipError_t launch_qknorm(int dtype, int n_tok, int H, int D, void* q, void* k, const NormArgs& norm,
                         hipStream_t stream);

hipError_t launch_rope(int dtype, int n_tok, int H, int D, void* q, void* k, const int32_t* pos,
                       const RopeArgs& rope, hipStream_t stream);

struct BuilderArgs {
    const int32_t* ord_frame;
    const int32_t* pending_frame;
    const int32_t* special_frame;
    int32_t* out;            // records, 5 int32 each
    int64_t n_key, n_special;
    int n_win, pending;
    int S, W, P, R, ns, cross, num_slots, n_ord;
    int total;               // records to write
};
hipError_t launch_builder(const BuilderArgs& a, hipStream_t stream);

hipError_t launch_mask(int F, int P, int W, int S, int token_level, uint8_t* out,
                       hipStream_t stream);

// Attention: bf16 on MFMA or fp32 on the vector ALUs.  Streaming bf16 runs
// p.ncols columns of p.qtiles work-groups (grid = ncols * qtiles); heads
// split across columns leave partials for launch_merge.  Streaming bf16
// with p.dseg != null reads the segments from device memory and uses the
// first min(p.ncols, H * tiles) columns.
hipError_t launch_attention(int dtype, int D, bool prefill, const AttnParams& p, int grid,
                            hipStream_t stream);
int attention_q_tile(int dtype);
// Work-groups of the streaming attention kernel that fit on one CU at once.
int attention_blocks_per_cu(int dtype, int D);

// Combine the streaming partials of heads split across columns (n = key
// tiles per head) into out [nq, H, D] bf16 and lse [H, nq] (may be null).
// dn != null: n is read from device memory and the columns clamped to H * n,
// as the attention kernel does with device segments.
hipError_t launch_merge(int D, int H, int nq, int n, int ncols, const float* part_o, const float* part_ml, void* out,
                        float* lse, int64_t rs, int64_t hs, const int* dn, hipStream_t stream);

// Token decode over rolling buffers ([H = sequences x kv heads][rows][D] and
// V^T): the streaming attention kernel with one wave per work-group, whose
// 32 query rows are the query heads of one kv group (p.nq <= 32).  With
// p.dk != null the new token (p.dk, p.dv: [H][D]) is written into row
// p.dslot of every buffer by the work-group that reads that row's tile,
// before its tile loads.
hipError_t launch_attention_decode(int D, const AttnParams& p, int grid, hipStream_t stream);
int attention_decode_blocks_per_cu(int D);
int attention_decode_q_rows();

}  // namespace swa
