// Host-side ring bookkeeping of one layer's frame cache.
//
// Rules (guide "Sliding Window Attention Mechanism in AggregatorStream",
// section "KV Cache Eviction Strategy"; explainer on akshathtiwari.co.in,
// rolling-buffer paragraph; FlashInferBlock.forward streaming branch):
//  * keyframe ordinal n (count of keyframes since reset) lives in page slot
//    n when n < S (scale frames, never evicted), otherwise in the rolling
//    window slot S + ((n - S) mod W);
//  * eviction drops cached positions [S, n_cached - W) once more than S + W
//    keyframes are cached; with cross-frame special retention each dropped
//    frame's special rows go to a FIFO ring of R entries (entry e in slot
//    e mod R);
//  * a non-keyframe sits in the scratch slot, with eviction deferred, until
//    it is rolled back;
//  * with the window off (W < 0) every keyframe stays, slot = n, up to a
//    capacity of max_frames.
// Keys are listed in ascending frame order: scale frames, retained special
// rows, window frames, the pending non-keyframe.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace swa {

struct RingConfig {
    int P = 0;              // tokens (rows) per frame
    int S = 0;              // scale frames
    int W = -1;             // window frames, -1 = off
    int max_frames = 0;     // capacity with the window off
    bool cross_special = false;
    int special_row0 = 0;
    int ns = 0;             // special rows per frame
    int R = 0;              // retained special entries
};

struct PageRec {
    int32_t frame, region, slot, row0, nrows;
};

struct RowSeg {
    int32_t lo, hi;         // rows [lo, hi) of the layer's row space
};

// What the device must do for one append.
struct AppendPlan {
    bool keyframe = true;
    int slot = 0;           // destination page slot
    int ord_index = -1;     // frame-id table entry of a keyframe (-1: pending)
    bool retain = false;    // copy the displaced frame's special rows first
    int victim_slot = 0;
    int special_slot = 0;   // ring entry (push index mod R)
    int special_id_index = 0;
    int64_t victim_frame = 0;
};

// Counters the device page-list builder needs.
struct RingCounters {
    int64_t n_key = 0;      // keyframes appended since reset
    int32_t n_win = 0;      // cached window frames
    int64_t n_special = 0;  // special entries pushed since reset
    int32_t pending = 0;    // a non-keyframe is pending
};

class Ring {
public:
    explicit Ring(const RingConfig& cfg);

    void reset();
    // 0 or a negative SWA_E_* code with *err set.
    int plan_append(int64_t t, bool keyframe, AppendPlan* plan, std::string* err) const;
    void commit_append(const AppendPlan& plan, int64_t t);
    int evict();            // number of dropped frames
    int rollback(std::string* err);

    void pages(std::vector<PageRec>* out) const;
    // Row segments of the visible keys in key order, adjacent ones merged.
    void segments(std::vector<RowSeg>* out) const;
    int64_t visible_rows() const;
    // A keyframe was appended to a full window and the eviction that makes
    // room for it has not run yet: the append has already overwritten the
    // page of the frame the eviction drops.
    bool eviction_pending() const { return cfg_.W >= 0 && n_win_ > cfg_.W; }

    RingCounters counters() const;
    int num_slots() const { return num_slots_; }
    int scratch_slot() const { return num_slots_ - 1; }
    int ord_table_size() const { return n_ord_; }
    int special_row_base() const { return num_slots_ * cfg_.P; }
    const RingConfig& config() const { return cfg_; }

    int slot_of(int64_t ordinal) const;
    int ord_index_of(int64_t ordinal) const;

private:
    int scale_cached() const;

    RingConfig cfg_;
    int num_slots_ = 0;
    int n_ord_ = 0;
    int64_t n_key_ = 0;
    int32_t n_win_ = 0;
    int64_t n_special_ = 0;
    bool pending_ = false;
    int64_t pending_frame_ = 0;
    bool has_last_ = false;
    int64_t last_frame_ = 0;
    std::vector<int64_t> ord_frame_;     // frame id per ordinal table entry
    std::vector<int64_t> special_frame_; // frame id per push index mod (R+1)
};

}  // namespace swa
