// Host-side ring bookkeeping; the rules are stated in ring.hpp.
#include "ring.hpp"

#include <algorithm>

#include "swa.h"

namespace swa {

Ring::Ring(const RingConfig& cfg) : cfg_(cfg) {
    if (cfg_.W >= 0) {
        num_slots_ = cfg_.S + cfg_.W + 1;          // + scratch
        n_ord_ = cfg_.S + cfg_.W + 1;              // one extra: a displaced frame keeps its id until evicted
    } else {
        num_slots_ = cfg_.max_frames + 1;
        n_ord_ = cfg_.max_frames;
    }
    ord_frame_.assign(n_ord_, -1);
    special_frame_.assign(cfg_.cross_special ? cfg_.R + 1 : 1, -1);
    reset();
}

void Ring::reset() {
    n_key_ = 0;
    n_win_ = 0;
    n_special_ = 0;
    pending_ = false;
    pending_frame_ = 0;
    has_last_ = false;
    last_frame_ = 0;
    std::fill(ord_frame_.begin(), ord_frame_.end(), -1);
    std::fill(special_frame_.begin(), special_frame_.end(), -1);
}

int Ring::slot_of(int64_t o) const {
    if (cfg_.W < 0 || o < cfg_.S) return static_cast<int>(o);
    return cfg_.S + static_cast<int>((o - cfg_.S) % cfg_.W);
}

int Ring::ord_index_of(int64_t o) const {
    if (cfg_.W < 0 || o < cfg_.S) return static_cast<int>(o);
    return cfg_.S + static_cast<int>((o - cfg_.S) % (cfg_.W + 1));
}

int Ring::scale_cached() const {
    if (cfg_.W < 0) return static_cast<int>(n_key_);
    return static_cast<int>(std::min<int64_t>(n_key_, cfg_.S));
}

int Ring::plan_append(int64_t t, bool keyframe, AppendPlan* plan, std::string* err) const {
    if (pending_) {
        *err = "a non-keyframe is pending; roll it back before the next append";
        return SWA_E_STATE;
    }
    if (eviction_pending()) {
        *err = "an eviction is pending; call kvcache_evict before the next append";
        return SWA_E_STATE;
    }
    if (has_last_ && t <= last_frame_) {
        *err = "frame index must increase within a stream";
        return SWA_E_INVAL;
    }
    if (t < 0 || t > INT32_MAX) {
        *err = "frame index out of range";
        return SWA_E_INVAL;
    }
    AppendPlan p;
    p.keyframe = keyframe;
    if (!keyframe) {
        p.slot = scratch_slot();
        p.ord_index = -1;
        *plan = p;
        return SWA_OK;
    }
    const int64_t o = n_key_;
    if (cfg_.W < 0 && o >= cfg_.max_frames) {
        *err = "cache full: window off and max_frames keyframes cached";
        return SWA_E_CAPACITY;
    }
    p.slot = slot_of(o);
    p.ord_index = ord_index_of(o);
    if (cfg_.W >= 0 && o >= cfg_.S && n_win_ == cfg_.W && cfg_.cross_special) {
        // The slot still holds the oldest window frame (ordinal o - W), which
        // the following eviction drops: keep its special rows first.
        const int64_t victim = o - cfg_.W;
        p.retain = true;
        p.victim_slot = slot_of(victim);
        p.victim_frame = ord_frame_[ord_index_of(victim)];
        p.special_slot = static_cast<int>(n_special_ % cfg_.R);
        p.special_id_index = static_cast<int>(n_special_ % (cfg_.R + 1));
    }
    *plan = p;
    return SWA_OK;
}

void Ring::commit_append(const AppendPlan& p, int64_t t) {
    has_last_ = true;
    last_frame_ = t;
    if (!p.keyframe) {
        pending_ = true;
        pending_frame_ = t;
        return;
    }
    if (p.retain) special_frame_[p.special_id_index] = p.victim_frame;
    ord_frame_[p.ord_index] = t;
    if (cfg_.W >= 0 && n_key_ >= cfg_.S) n_win_ += 1;
    n_key_ += 1;
}

int Ring::evict() {
    if (cfg_.W < 0 || pending_) return 0;        // window off / eviction deferred
    const int n_cached = scale_cached() + n_win_;
    if (n_cached <= cfg_.W + cfg_.S) return 0;
    // positions [S, n_cached - W) are the oldest window frames
    const int drop = n_cached - cfg_.W - cfg_.S;
    if (cfg_.cross_special) n_special_ += drop;
    n_win_ -= drop;
    return drop;
}

int Ring::rollback(std::string* err) {
    if (!pending_) {
        *err = "nothing to roll back: no non-keyframe is pending";
        return SWA_E_STATE;
    }
    pending_ = false;
    return SWA_OK;
}

void Ring::pages(std::vector<PageRec>* out) const {
    out->clear();
    const int P = cfg_.P;
    const int sc = scale_cached();
    for (int o = 0; o < sc; ++o)
        out->push_back({static_cast<int32_t>(ord_frame_[ord_index_of(o)]), SWA_REGION_FRAME,
                        slot_of(o), 0, P});
    if (cfg_.cross_special) {
        const int64_t e0 = std::max<int64_t>(0, n_special_ - cfg_.R);
        for (int64_t e = e0; e < n_special_; ++e) {
            const int s = static_cast<int>(e % cfg_.R);
            out->push_back({static_cast<int32_t>(special_frame_[e % (cfg_.R + 1)]),
                            SWA_REGION_SPECIAL, s, s * cfg_.ns, cfg_.ns});
        }
    }
    for (int64_t o = n_key_ - n_win_; o < n_key_; ++o)
        out->push_back({static_cast<int32_t>(ord_frame_[ord_index_of(o)]), SWA_REGION_FRAME,
                        slot_of(o), 0, P});
    if (pending_)
        out->push_back({static_cast<int32_t>(pending_frame_), SWA_REGION_FRAME, scratch_slot(), 0, P});
}

void Ring::segments(std::vector<RowSeg>* out) const {
    out->clear();
    const int P = cfg_.P;
    auto push = [out](int lo, int hi) {
        if (hi <= lo) return;
        if (!out->empty() && out->back().hi == lo)
            out->back().hi = hi;
        else
            out->push_back({lo, hi});
    };
    push(0, scale_cached() * P);
    if (cfg_.cross_special && n_special_ > 0) {
        const int base = special_row_base();
        const int64_t e0 = std::max<int64_t>(0, n_special_ - cfg_.R);
        const int n = static_cast<int>(n_special_ - e0);
        const int first = static_cast<int>(e0 % cfg_.R);
        const int run1 = std::min(n, cfg_.R - first);
        push(base + first * cfg_.ns, base + (first + run1) * cfg_.ns);
        push(base, base + (n - run1) * cfg_.ns);
    }
    if (n_win_ > 0) {
        const int64_t o0 = n_key_ - n_win_;
        const int first = static_cast<int>((o0 - cfg_.S) % cfg_.W);
        const int run1 = std::min(n_win_, cfg_.W - first);
        push((cfg_.S + first) * P, (cfg_.S + first + run1) * P);
        push(cfg_.S * P, (cfg_.S + n_win_ - run1) * P);
    }
    if (pending_) push(scratch_slot() * P, (scratch_slot() + 1) * P);
}

int64_t Ring::visible_rows() const {
    std::vector<RowSeg> segs;
    segments(&segs);
    int64_t n = 0;
    for (const auto& s : segs) n += s.hi - s.lo;
    return n;
}

RingCounters Ring::counters() const {
    RingCounters c;
    c.n_key = n_key_;
    c.n_win = n_win_;
    c.n_special = n_special_;
    c.pending = pending_ ? 1 : 0;
    return c;
}

}  // namespace swa
