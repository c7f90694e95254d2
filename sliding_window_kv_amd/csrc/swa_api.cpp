// C ABI of the library (declared in include/swa.h): argument checks, the
// cache's pool layout, host ring bookkeeping and kernel orchestration.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <type_traits>
#include <vector>

#include "api_internal.hpp"
#include "launch.hpp"
#include "ring.hpp"
#include "swa.h"

static_assert(std::is_same<swa_stream_t, hipStream_t>::value, "swa_stream_t must be hipStream_t");

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
    g_err = msg;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(SWA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

struct Layout {
    int P, H, D, elem, W, S, num_slots, n_ord, nspid, R, ns, rows, special_row_base;
    int max_records;
    int64_t k_bytes, v_bytes, meta_bytes, layer_bytes, work_offset, work_bytes;
    int64_t meta_pending, meta_special, meta_records;   // int32 offsets inside meta
    int64_t plan_offset;                                 // device step plan (captured steps), in the work area
    int64_t total_bytes;
    int64_t part_o_floats;                               // floats of the O partials
};

// Element offsets inside one head's K or V^T region are 32-bit ints in the
// kernels (and byte offsets twice that): keep D * rows * element size below
// 2^31.
bool row_space_fits(int64_t used_rows, int D, int elem) {
    const int64_t rows = (used_rows + 64 + 63) / 64 * 64;
    return rows * D * elem < (int64_t(1) << 31);
}

int check_config(const swa_config* c, std::string* err) {
    if (c == nullptr) return *err = "null config", SWA_E_INVAL;
    if (c->num_layers < 1) return *err = "num_layers must be >= 1", SWA_E_INVAL;
    if (c->tokens_per_frame < 1 || c->tokens_per_frame > (1 << 20))
        return *err = "tokens_per_frame out of range", SWA_E_INVAL;
    if (c->num_heads < 1 || c->num_heads > 1024) return *err = "num_heads out of range", SWA_E_INVAL;
    if (c->head_dim != 32 && c->head_dim != 64) return *err = "head_dim must be 32 or 64", SWA_E_UNSUPPORTED;
    if (c->dtype != SWA_BF16 && c->dtype != SWA_F32) return *err = "dtype must be SWA_BF16 or SWA_F32", SWA_E_INVAL;
    if (c->sliding_window_size == 0 || c->sliding_window_size < -1)
        return *err = "sliding_window_size must be -1 or positive", SWA_E_INVAL;
    if (c->num_frame_per_block < 1) return *err = "num_frame_per_block must be >= 1", SWA_E_INVAL;
    if (c->scale_frames < 0) return *err = "scale_frames must be >= 0", SWA_E_INVAL;
    if (c->sliding_window_size == -1 && c->max_frames < 1)
        return *err = "max_frames must be >= 1 when the window is off", SWA_E_INVAL;
    if (c->cross_frame_special) {
        if (c->special_rows < 1 || c->special_row0 < 0 ||
            c->special_row0 + c->special_rows > c->tokens_per_frame)
            return *err = "special rows must lie inside a frame", SWA_E_INVAL;
        if (c->max_special_frames < 1) return *err = "max_special_frames must be >= 1", SWA_E_INVAL;
    }
    const int64_t W = c->sliding_window_size == -1
                          ? -1
                          : static_cast<int64_t>(c->sliding_window_size) * c->num_frame_per_block;
    const int64_t slots = W >= 0 ? c->scale_frames + W + 1 : c->max_frames + 1;
    const int64_t sp = c->cross_frame_special ? static_cast<int64_t>(c->max_special_frames) * c->special_rows : 0;
    if (slots * c->tokens_per_frame + sp + 128 > (1ll << 30) || W > (1 << 24))
        return *err = "cache row space too large", SWA_E_INVAL;
    if (!row_space_fits(slots * c->tokens_per_frame + sp, c->head_dim, c->dtype == SWA_BF16 ? 2 : 4))
        return *err = "cache row space too large: one head's region must stay below 2 GiB", SWA_E_INVAL;
    const int pairs = c->rope_pairs_t + c->rope_pairs_h + c->rope_pairs_w;
    if (pairs != 0 && (pairs != c->head_dim / 2 || c->rope_pairs_t < 0 || c->rope_pairs_h < 0 ||
                       c->rope_pairs_w < 0 || !(c->rope_theta > 0.f)))
        return *err = "rope bands must add up to head_dim/2 with theta > 0", SWA_E_INVAL;
    return SWA_OK;
}

Layout make_layout(const swa_config* c) {
    Layout L{};
    L.P = c->tokens_per_frame;
    L.H = c->num_heads;
    L.D = c->head_dim;
    L.elem = c->dtype == SWA_BF16 ? 2 : 4;
    L.W = c->sliding_window_size == -1 ? -1 : c->sliding_window_size * c->num_frame_per_block;
    L.S = c->scale_frames;
    L.num_slots = L.W >= 0 ? L.S + L.W + 1 : c->max_frames + 1;
    L.n_ord = L.W >= 0 ? L.S + L.W + 1 : c->max_frames;
    L.R = c->cross_frame_special ? c->max_special_frames : 0;
    L.ns = c->cross_frame_special ? c->special_rows : 0;
    L.nspid = c->cross_frame_special ? L.R + 1 : 1;
    L.special_row_base = L.num_slots * L.P;
    L.rows = static_cast<int>(align_up(static_cast<int64_t>(L.special_row_base) + int64_t(L.R) * L.ns + 64, 64));
    L.max_records = L.num_slots + L.R;
    L.k_bytes = align_up(int64_t(L.H) * L.rows * L.D * L.elem, 256);
    L.v_bytes = L.k_bytes;
    L.meta_pending = L.n_ord;
    L.meta_special = L.n_ord + 1;
    L.meta_records = align_up(L.meta_special + L.nspid, 4);
    L.meta_bytes = align_up((L.meta_records + int64_t(L.max_records) * 5) * 4, 256);
    L.layer_bytes = L.k_bytes + L.v_bytes + L.meta_bytes;
    L.work_offset = L.layer_bytes * c->num_layers;
    if (c->dtype == SWA_BF16) {
        const int64_t pieces = 2 * int64_t(swa::kMaxCols);   // two partial slots per column
        L.part_o_floats = pieces * L.P * L.D;
        L.work_bytes = align_up(L.part_o_floats * 4, 256) + align_up(pieces * L.P * 2 * 4, 256);
        L.plan_offset = L.work_offset + L.work_bytes;
        L.work_bytes += align_up(sizeof(swa::StepPlan), 256);
    } else {
        L.part_o_floats = 0;
        L.work_bytes = 0;
        L.plan_offset = -1;
    }
    L.total_bytes = L.work_offset + L.work_bytes;
    return L;
}

swa::RingConfig ring_config(const swa_config* c, const Layout& L) {
    swa::RingConfig r;
    r.P = L.P;
    r.S = L.S;
    r.W = L.W;
    r.max_frames = c->max_frames;
    r.cross_special = c->cross_frame_special != 0;
    r.special_row0 = c->special_row0;
    r.ns = L.ns;
    r.R = L.R;
    return r;
}

void make_rope(int pt, int ph, int pw, float theta, swa::RopeArgs* r) {
    std::memset(r, 0, sizeof(*r));
    r->pairs_t = pt;
    r->pairs_h = ph;
    r->pairs_w = pw;
    const int bands[3] = {pt, ph, pw};
    int p = 0;
    for (int b = 0; b < 3; ++b)
        for (int kk = 0; kk < bands[b]; ++kk)
            r->freq[p++] = std::pow(static_cast<double>(theta), -static_cast<double>(kk) / bands[b]);
}

// Key tiles of a row segment: 64 rows each, the first starting on a 64-row boundary.
int tiles_of(int lo, int hi) { return (hi - (lo & ~63) + 63) / 64; }

}  // namespace

struct swa_cache {
    swa_config cfg;
    Layout L;
    char* pool = nullptr;
    bool dry = false;
    int splits = 0;          // 0 = automatic
    int num_cus = 256;
    int blocks_per_cu = 1;   // resident attention work-groups per CU
    std::vector<swa::Ring> rings;
    swa::RopeArgs rope;

    char* layer_base(int l) const { return pool + int64_t(l) * L.layer_bytes; }
    void* kreg(int l) const { return layer_base(l); }
    void* vreg(int l) const { return layer_base(l) + L.k_bytes; }
    int32_t* meta(int l) const { return reinterpret_cast<int32_t*>(layer_base(l) + L.k_bytes + L.v_bytes); }
    float* part_o() const { return reinterpret_cast<float*>(pool + L.work_offset); }
    float* part_ml() const {
        return reinterpret_cast<float*>(pool + L.work_offset + align_up(L.part_o_floats * 4, 256));
    }
    swa::StepPlan* step_plan() const { return reinterpret_cast<swa::StepPlan*>(pool + L.plan_offset); }
};

// A captured streaming step of every layer (swa_graph_create).
struct swa_graph {
    swa_cache* c = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    ~swa_graph() {
        if (exec != nullptr) (void)hipGraphExecDestroy(exec);
        if (graph != nullptr) (void)hipGraphDestroy(graph);
    }
};

namespace {

int check_layer(const swa_cache* c, int layer) {
    if (c == nullptr) return fail(SWA_E_INVAL, "null cache");
    if (layer < 0 || layer >= c->cfg.num_layers) return fail(SWA_E_INVAL, "layer index out of range");
    return SWA_OK;
}

// Columns of one streaming attention call (each runs as qtiles work-groups
// over an equal share of the H * n (head, key tile) space).  Automatic: as
// many as the GPU holds at once, so the launch is one balanced round;
// splits = k: every head cut into k equal pieces (k = 1: no partials).
int pick_columns(const swa_cache* c, int qtiles, int n) {
    const int64_t hn = int64_t(c->L.H) * n;
    int64_t cols;
    if (c->splits > 0)
        cols = int64_t(c->L.H) * c->splits;
    else
        cols = std::max(1, c->num_cus * c->blocks_per_cu / std::max(1, qtiles));
    cols = std::min<int64_t>(cols, swa::kMaxCols);
    cols = std::min<int64_t>(cols, hn);
    return static_cast<int>(std::max<int64_t>(cols, 1));
}

// Enqueue the device side of one append: one launch that retains the special
// rows of the slot's previous occupant (if it is evicted) and then copies the
// frame in, with optional norm and RoPE.
int enqueue_append(swa_cache* c, int layer, const swa::AppendPlan& plan, int64_t t, void* q,
                   const void* k, const void* v, const int32_t* pos, const swa::NormArgs* norm,
                   hipStream_t stream) {
    const Layout& L = c->L;
    const int dt = c->cfg.dtype;
    swa::RetainArgs ret{0, 0, 0, nullptr, 0};
    if (plan.retain) {                       // the slot's occupant is evicted: its special rows go first
        ret.src_row = plan.victim_slot * L.P + c->cfg.special_row0;
        ret.dst_row = L.special_row_base + plan.special_slot * L.ns;
        ret.ns = L.ns;
        ret.meta = c->meta(layer) + L.meta_special + plan.special_id_index;
        ret.frame = static_cast<int32_t>(plan.victim_frame);
    }
    int32_t* slot_meta = plan.keyframe ? c->meta(layer) + plan.ord_index : c->meta(layer) + L.meta_pending;
    hipError_t e = swa::launch_append(dt, L.H, L.D, L.P, plan.slot * L.P, L.rows, k, v, c->kreg(layer),
                                      c->vreg(layer), q, pos, pos != nullptr ? &c->rope : nullptr, norm, slot_meta,
                                      static_cast<int32_t>(t), ret, nullptr, stream);
    if (e != hipSuccess) return hip_fail(e, "append kernel launch");
    return SWA_OK;
}

// The ring's visible rows as the kernels' segment list (tiles numbered
// across segments in key order).
int fill_segs(const swa::Ring& ring, swa::SegList* out) {
    std::vector<swa::RowSeg> segs;
    ring.segments(&segs);
    if (segs.size() > static_cast<size_t>(swa::kMaxSegs)) return fail(SWA_E_STATE, "internal: bad segment list");
    if (segs.empty()) return fail(SWA_E_STATE, "no cached frame to attend to");
    out->n = static_cast<int>(segs.size());
    int tiles = 0;
    for (int i = 0; i < swa::kMaxSegs; ++i) {
        if (i < out->n) {
            out->lo[i] = segs[i].lo;
            out->hi[i] = segs[i].hi;
            out->tile0[i] = tiles;
            tiles += tiles_of(segs[i].lo, segs[i].hi);
        } else {
            out->lo[i] = out->hi[i] = 0;
            out->tile0[i] = 1 << 30;
        }
    }
    out->total_tiles = tiles;
    return SWA_OK;
}

// Attention parameters of one layer's frame query (everything but the
// segments and the column count).
swa::AttnParams frame_attn_params(const swa_cache* c, int layer, const void* q, void* out, float* lse) {
    const Layout& L = c->L;
    swa::AttnParams p{};
    p.q = q;
    p.kreg = c->kreg(layer);
    p.vreg = c->vreg(layer);
    p.out = out;
    p.lse = lse;
    p.nq = L.P;
    p.H = L.H;
    p.rs = int64_t(L.H) * L.D;
    p.hs = L.D;
    p.rows = L.rows;
    p.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(L.D)));
    p.F = 1;
    const int qrows = swa::attention_q_tile(c->cfg.dtype);
    p.qtiles = (L.P + qrows - 1) / qrows;
    if (c->cfg.dtype == SWA_BF16) {
        p.part_o = c->part_o();
        p.part_ml = c->part_ml();
    }
    return p;
}

// Attention of q over the layer's visible rows (split-KV + combine for bf16).
int enqueue_attention(swa_cache* c, int layer, const void* q, void* out, float* lse, hipStream_t stream) {
    const Layout& L = c->L;
    swa::AttnParams p = frame_attn_params(c, layer, q, out, lse);
    const int rc = fill_segs(c->rings[layer], &p.seg);
    if (rc != SWA_OK) return rc;
    const int tiles = p.seg.total_tiles;
    p.ncols = c->cfg.dtype == SWA_BF16 ? pick_columns(c, p.qtiles, tiles) : 1;
    hipError_t e = swa::launch_attention(c->cfg.dtype, L.D, false, p, p.ncols * p.qtiles, stream);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    // every head inside one column (ncols divides H): no partials to merge
    if (c->cfg.dtype == SWA_BF16 && !(p.ncols <= L.H && L.H % p.ncols == 0)) {
        e = swa::launch_merge(L.D, L.H, L.P, tiles, p.ncols, p.part_o, p.part_ml, out, lse, p.rs, p.hs, nullptr,
                              stream);
        if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    }
    return SWA_OK;
}

// One layer's step with every ring-dependent value read from the device
// step plan, for capture: append (+ retention if the plan asks, + norm,
// + RoPE), attention over the plan's segments on a fixed number of
// columns, merge.
int enqueue_planned_layer(swa_cache* c, int layer, void* q, const void* k, const void* v, const int32_t* pos,
                          const swa::NormArgs* norm, void* out, float* lse, hipStream_t stream) {
    const Layout& L = c->L;
    const int dt = c->cfg.dtype;
    const swa::StepPlan* plan = c->step_plan();
    // retention (if the plan asks) happens inside the append
    const swa::RetainArgs ret{0, 0, c->cfg.cross_frame_special ? L.ns : 0, nullptr, 0};
    hipError_t e = swa::launch_append(dt, L.H, L.D, L.P, 0, L.rows, k, v, c->kreg(layer), c->vreg(layer), q, pos,
                                      pos != nullptr ? &c->rope : nullptr, norm, c->meta(layer), 0, ret, plan, stream);
    if (e != hipSuccess) return hip_fail(e, "append kernel launch");
    swa::AttnParams p = frame_attn_params(c, layer, q, out, lse);
    p.dseg = &plan->seg;
    // the automatic (or fixed-split) column count before the clamp to the
    // tile space, which the kernels apply on the device
    p.ncols = static_cast<int>(std::min<int64_t>(
        c->splits > 0 ? int64_t(L.H) * c->splits : std::max(1, c->num_cus * c->blocks_per_cu / std::max(1, p.qtiles)),
        swa::kMaxCols));
    e = swa::launch_attention(dt, L.D, false, p, p.ncols * p.qtiles, stream);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    if (!(p.ncols <= L.H && L.H % p.ncols == 0)) {
        e = swa::launch_merge(L.D, L.H, L.P, 1, p.ncols, p.part_o, p.part_ml, out, lse, p.rs, p.hs,
                              &plan->seg.total_tiles, stream);
        if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    }
    return SWA_OK;
}

}  // namespace

extern "C" {

size_t swa_cache_pool_bytes(const swa_config* cfg) {
    std::string err;
    if (check_config(cfg, &err) != SWA_OK) {
        g_err = err;
        return 0;
    }
    return static_cast<size_t>(make_layout(cfg).total_bytes);
}

int swa_cache_create(const swa_config* cfg, void* dev_pool, size_t pool_bytes, swa_cache** out) {
    if (out == nullptr) return fail(SWA_E_INVAL, "null output handle");
    *out = nullptr;
    std::string err;
    const int rc = check_config(cfg, &err);
    if (rc != SWA_OK) return fail(rc, err);
    const Layout L = make_layout(cfg);
    const bool dry = dev_pool == nullptr && pool_bytes == 0;
    if (!dry) {
        if (dev_pool == nullptr) return fail(SWA_E_INVAL, "null pool with nonzero size");
        if (reinterpret_cast<uintptr_t>(dev_pool) % 256 != 0) return fail(SWA_E_INVAL, "pool must be 256-byte aligned");
        if (pool_bytes < static_cast<size_t>(L.total_bytes))
            return fail(SWA_E_INVAL, "pool smaller than swa_cache_pool_bytes()");
    }
    swa_cache* c = new (std::nothrow) swa_cache();
    if (c == nullptr) return fail(SWA_E_INVAL, "out of host memory");
    c->cfg = *cfg;
    c->L = L;
    c->pool = static_cast<char*>(dev_pool);
    c->dry = dry;
    const swa::RingConfig rc2 = ring_config(cfg, L);
    c->rings.reserve(cfg->num_layers);
    for (int i = 0; i < cfg->num_layers; ++i) c->rings.emplace_back(rc2);
    make_rope(cfg->rope_pairs_t, cfg->rope_pairs_h, cfg->rope_pairs_w, cfg->rope_theta, &c->rope);
    if (!dry) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess &&
            prop.multiProcessorCount > 0)
            c->num_cus = prop.multiProcessorCount;
        c->blocks_per_cu = swa::attention_blocks_per_cu(cfg->dtype, cfg->head_dim);
    }
    *out = c;
    return SWA_OK;
}

int swa_cache_destroy(swa_cache* cache) {
    delete cache;
    return SWA_OK;
}

int swa_cache_layout(const swa_cache* c, swa_layout* out) {
    if (c == nullptr || out == nullptr) return fail(SWA_E_INVAL, "null argument");
    const Layout& L = c->L;
    out->layer_bytes = L.layer_bytes;
    out->k_offset = 0;
    out->v_offset = L.k_bytes;
    out->meta_offset = L.k_bytes + L.v_bytes;
    out->work_offset = L.work_offset;
    out->work_bytes = L.work_bytes;
    out->rows = L.rows;
    out->num_slots = L.num_slots;
    out->special_row_base = L.special_row_base;
    out->elem_bytes = L.elem;
    out->window_frames = L.W;
    out->scratch_slot = L.num_slots - 1;
    return SWA_OK;
}

int swa_cache_set_splits(swa_cache* c, int splits) {
    if (c == nullptr) return fail(SWA_E_INVAL, "null cache");
    if (splits < 0 || splits > swa::kMaxCols) return fail(SWA_E_INVAL, "splits must be 0..256");
    c->splits = splits;
    return SWA_OK;
}

int kvcache_reset(swa_cache* c, swa_stream_t) {
    if (c == nullptr) return fail(SWA_E_INVAL, "null cache");
    for (auto& r : c->rings) r.reset();
    return SWA_OK;
}

int kvcache_append(swa_cache* c, int layer, int64_t t, const void* k, const void* v, int keyframe,
                   swa_stream_t stream) {
    int rc = check_layer(c, layer);
    if (rc != SWA_OK) return rc;
    if (!c->dry && (k == nullptr || v == nullptr)) return fail(SWA_E_INVAL, "null k or v");
    swa::AppendPlan plan;
    std::string err;
    rc = c->rings[layer].plan_append(t, keyframe != 0, &plan, &err);
    if (rc != SWA_OK) return fail(rc, err);
    if (!c->dry) {
        rc = enqueue_append(c, layer, plan, t, nullptr, k, v, nullptr, nullptr, stream);
        if (rc != SWA_OK) return rc;
    }
    c->rings[layer].commit_append(plan, t);
    return SWA_OK;
}

int kvcache_evict(swa_cache* c, int layer, swa_stream_t) {
    const int rc = check_layer(c, layer);
    if (rc != SWA_OK) return rc;
    c->rings[layer].evict();
    return SWA_OK;
}

int kvcache_rollback(swa_cache* c, int layer, swa_stream_t) {
    int rc = check_layer(c, layer);
    if (rc != SWA_OK) return rc;
    std::string err;
    rc = c->rings[layer].rollback(&err);
    if (rc != SWA_OK) return fail(rc, err);
    return SWA_OK;
}

int kvcache_attend(swa_cache* c, int layer, const void* q, void* out, float* lse, swa_stream_t stream) {
    const int rc = check_layer(c, layer);
    if (rc != SWA_OK) return rc;
    if (c->rings[layer].eviction_pending())
        return fail(SWA_E_STATE, "an eviction is pending; call kvcache_evict before attending");
    if (c->dry) return fail(SWA_E_STATE, "bookkeeping-only cache cannot attend");
    if (q == nullptr || out == nullptr) return fail(SWA_E_INVAL, "null tensor");
    return enqueue_attention(c, layer, q, out, lse, stream);
}

int kvcache_visible_pages(const swa_cache* c, int layer, swa_page* out, int cap, int* n_out) {
    const int rc = check_layer(c, layer);
    if (rc != SWA_OK) return rc;
    if (n_out == nullptr || cap < 0 || (cap > 0 && out == nullptr)) return fail(SWA_E_INVAL, "bad output buffer");
    std::vector<swa::PageRec> recs;
    c->rings[layer].pages(&recs);
    *n_out = static_cast<int>(recs.size());
    const int n = std::min<int>(cap, static_cast<int>(recs.size()));
    for (int i = 0; i < n; ++i) {
        out[i].frame = recs[i].frame;
        out[i].region = recs[i].region;
        out[i].slot = recs[i].slot;
        out[i].row0 = recs[i].row0;
        out[i].nrows = recs[i].nrows;
    }
    return SWA_OK;
}

int kvcache_read_device_pages(swa_cache* c, int layer, swa_page* host_out, int cap, int* n_out,
                              swa_stream_t stream) {
    int rc = check_layer(c, layer);
    if (rc != SWA_OK) return rc;
    if (c->rings[layer].eviction_pending())
        return fail(SWA_E_STATE, "an eviction is pending; call kvcache_evict before reading the page list");
    if (c->dry) return fail(SWA_E_STATE, "bookkeeping-only cache has no device state");
    if (n_out == nullptr || cap < 0 || (cap > 0 && host_out == nullptr)) return fail(SWA_E_INVAL, "bad output buffer");
    const swa::Ring& ring = c->rings[layer];
    const swa::RingCounters cnt = ring.counters();
    std::vector<swa::PageRec> recs;
    ring.pages(&recs);
    const int total = static_cast<int>(recs.size());
    *n_out = total;
    if (total == 0) return SWA_OK;
    const Layout& L = c->L;
    int32_t* meta = c->meta(layer);
    swa::BuilderArgs a{};
    a.ord_frame = meta;
    a.pending_frame = meta + L.meta_pending;
    a.special_frame = meta + L.meta_special;
    a.out = meta + L.meta_records;
    a.n_key = cnt.n_key;
    a.n_special = cnt.n_special;
    a.n_win = cnt.n_win;
    a.pending = cnt.pending;
    a.S = L.S;
    a.W = L.W;
    a.P = L.P;
    a.R = L.R;
    a.ns = L.ns;
    a.cross = c->cfg.cross_frame_special ? 1 : 0;
    a.num_slots = L.num_slots;
    a.n_ord = L.n_ord;
    a.total = total;
    hipError_t e = swa::launch_builder(a, stream);
    if (e != hipSuccess) return hip_fail(e, "page-list builder launch");
    std::vector<int32_t> buf(size_t(total) * 5);
    e = hipMemcpyAsync(buf.data(), a.out, buf.size() * 4, hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess) return hip_fail(e, "page-list copy");
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    const int n = std::min(cap, total);
    for (int i = 0; i < n; ++i) {
        host_out[i].frame = buf[5 * i];
        host_out[i].region = buf[5 * i + 1];
        host_out[i].slot = buf[5 * i + 2];
        host_out[i].row0 = buf[5 * i + 3];
        host_out[i].nrows = buf[5 * i + 4];
    }
    return SWA_OK;
}

int rope3d_apply(void* q, void* k, const int32_t* pos, int n_tokens, int H, int D, int pt, int ph, int pw,
                 float theta, int dtype, swa_stream_t stream) {
    if (pos == nullptr || (q == nullptr && k == nullptr)) return fail(SWA_E_INVAL, "null pointer");
    if (n_tokens < 0 || H < 1) return fail(SWA_E_INVAL, "bad shape");
    if (D != 32 && D != 64) return fail(SWA_E_UNSUPPORTED, "head_dim must be 32 or 64");
    if (dtype != SWA_BF16 && dtype != SWA_F32) return fail(SWA_E_INVAL, "bad dtype");
    if (pt < 0 || ph < 0 || pw < 0 || pt + ph + pw != D / 2 || !(theta > 0.f))
        return fail(SWA_E_INVAL, "rope bands must add up to head_dim/2 with theta > 0");
    if (n_tokens == 0) return SWA_OK;
    swa::RopeArgs r;
    make_rope(pt, ph, pw, theta, &r);
    hipError_t e = swa::launch_rope(dtype, n_tokens, H, D, q, k, pos, r, stream);
    if (e != hipSuccess) return hip_fail(e, "rope kernel launch");
    return SWA_OK;
}

}  // extern "C"

namespace {

using swa::kMaxDecodeCols;

struct DecodeLayout {
    int64_t rows, k_bytes, total;            // K and V^T regions of the rolling buffers
};

DecodeLayout decode_layout(int B, int Hkv, int W, int D) {
    DecodeLayout d;
    d.rows = align_up(int64_t(W) + 64, 64);
    d.k_bytes = align_up(int64_t(B) * Hkv * d.rows * D * 2, 256);
    d.total = 2 * d.k_bytes;
    return d;
}

int64_t decode_work_bytes(int G, int D) { return swa::decode_partials_bytes(G, D, kMaxDecodeCols); }

// Resident decode work-groups on the current device (cached per device).
int decode_fit(int D) {
    static int cached[2][64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int& f = cached[D == 64 ? 1 : 0][dev];
    if (f == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        f = cus * swa::attention_decode_blocks_per_cu(D);
    }
    return f;
}

int stream_step(swa_cache* c, int layer, int64_t t, void* q, const void* k, const void* v, const int32_t* pos,
                const swa::NormArgs* norm, int keyframe, void* out, float* lse, swa_stream_t stream) {
    int rc = check_layer(c, layer);
    if (rc != SWA_OK) return rc;
    if (c->dry) return fail(SWA_E_STATE, "bookkeeping-only cache cannot attend");
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return fail(SWA_E_INVAL, "null tensor");
    if (pos != nullptr && c->cfg.rope_pairs_t + c->cfg.rope_pairs_h + c->cfg.rope_pairs_w == 0)
        return fail(SWA_E_INVAL, "positions given but the config has no rope bands");
    swa::Ring& ring = c->rings[layer];
    swa::AppendPlan plan;
    std::string err;
    rc = ring.plan_append(t, keyframe != 0, &plan, &err);
    if (rc != SWA_OK) return fail(rc, err);
    rc = enqueue_append(c, layer, plan, t, q, k, v, pos, norm, stream);
    if (rc != SWA_OK) return rc;
    ring.commit_append(plan, t);
    if (keyframe) ring.evict();

    rc = enqueue_attention(c, layer, q, out, lse, stream);
    if (rc != SWA_OK) return rc;
    if (!keyframe) {
        rc = ring.rollback(&err);
        if (rc != SWA_OK) return fail(rc, err);
    }
    return SWA_OK;
}

}  // namespace

extern "C" {

int swa_stream_step(swa_cache* c, int layer, int64_t t, void* q, const void* k, const void* v,
                    const int32_t* pos, int keyframe, void* out, float* lse, swa_stream_t stream) {
    return stream_step(c, layer, t, q, k, v, pos, nullptr, keyframe, out, lse, stream);
}

int swa_stream_step_normed(swa_cache* c, int layer, int64_t t, void* q, const void* k, const void* v,
                           const float* qk_norm_weights, float eps, const int32_t* pos, int keyframe, void* out,
                           float* lse, swa_stream_t stream) {
    if (qk_norm_weights == nullptr) return fail(SWA_E_INVAL, "null norm weights");
    if (!(eps >= 0.f)) return fail(SWA_E_INVAL, "norm epsilon must be >= 0");
    const swa::NormArgs norm{qk_norm_weights, eps};
    return stream_step(c, layer, t, q, k, v, pos, &norm, keyframe, out, lse, stream);
}

int qk_norm_apply(void* q, void* k, int n_tokens, int H, int D, const float* weights, float eps, int dtype,
                  swa_stream_t stream) {
    if (weights == nullptr || (q == nullptr && k == nullptr)) return fail(SWA_E_INVAL, "null pointer");
    if (n_tokens < 0 || H < 1) return fail(SWA_E_INVAL, "bad shape");
    if (D != 32 && D != 64) return fail(SWA_E_UNSUPPORTED, "head_dim must be 32 or 64");
    if (dtype != SWA_BF16 && dtype != SWA_F32) return fail(SWA_E_INVAL, "bad dtype");
    if (!(eps >= 0.f)) return fail(SWA_E_INVAL, "norm epsilon must be >= 0");
    if (n_tokens == 0) return SWA_OK;
    hipError_t e = swa::launch_qknorm(dtype, n_tokens, H, D, q, k, swa::NormArgs{weights, eps}, stream);
    if (e != hipSuccess) return hip_fail(e, "norm kernel launch");
    return SWA_OK;
}

size_t swa_decode_cache_bytes(int B, int Hkv, int W, int D) {
    if (B < 1 || Hkv < 1 || W < 1 || (D != 32 && D != 64)) return 0;
    if (int64_t(W) + 128 > (1ll << 30) || !row_space_fits(W, D, 2)) return 0;
    return static_cast<size_t>(decode_layout(B, Hkv, W, D).total);
}

size_t swa_decode_workspace_bytes(int Hq, int Hkv, int D) {
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Hq / Hkv > swa::attention_decode_q_rows() || (D != 32 && D != 64))
        return 0;
    return static_cast<size_t>(decode_work_bytes(Hq / Hkv, D));
}

int swa_decode_step(void* cache, size_t cache_bytes, int B, int Hq, int Hkv, int W, int D, int64_t pos,
                    const void* q, const void* k, const void* v, void* out, float* lse, void* work,
                    size_t work_bytes, swa_stream_t stream) {
    if (work == nullptr) return fail(SWA_E_INVAL, "null pointer");
    if (Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 && (D == 32 || D == 64) &&
        work_bytes < static_cast<size_t>(decode_work_bytes(Hq / Hkv, D)))
        return fail(SWA_E_INVAL, "workspace smaller than swa_decode_workspace_bytes()");
    if (reinterpret_cast<uintptr_t>(work) % 256 != 0) return fail(SWA_E_INVAL, "workspace must be 256-byte aligned");
    return swa::decode_step_impl(cache, cache_bytes, B, Hq, Hkv, W, D, pos, q, k, v, out, lse, work, kMaxDecodeCols,
                                 stream);
}

size_t swa_prefill_workspace_bytes(int F, int P, int H, int D, int dtype) {
    if (F < 1 || P < 1 || H < 1 || (D != 32 && D != 64) || (dtype != SWA_BF16 && dtype != SWA_F32)) return 0;
    if (int64_t(F) * P + 128 > (1ll << 30) || !row_space_fits(int64_t(F) * P, D, dtype == SWA_BF16 ? 2 : 4)) return 0;
    const int64_t rows = align_up(int64_t(F) * P + 64, 64);
    const int64_t elem = dtype == SWA_BF16 ? 2 : 4;
    return static_cast<size_t>(2 * align_up(int64_t(H) * rows * D * elem, 256));
}

int swa_prefill_masked(const void* q, const void* k, const void* v, int F, int P, int H, int D, int sws,
                       int nfpb, int S, int dtype, void* out, float* lse, void* ws, size_t ws_bytes,
                       swa_stream_t stream) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return fail(SWA_E_INVAL, "null tensor");
    if (F < 1 || P < 1 || H < 1) return fail(SWA_E_INVAL, "F, P and H must be >= 1");
    if (int64_t(F) * P + 128 > (1ll << 30)) return fail(SWA_E_INVAL, "too many tokens");
    if (D != 32 && D != 64) return fail(SWA_E_UNSUPPORTED, "head_dim must be 32 or 64");
    if (dtype != SWA_BF16 && dtype != SWA_F32) return fail(SWA_E_INVAL, "bad dtype");
    if (!row_space_fits(int64_t(F) * P, D, dtype == SWA_BF16 ? 2 : 4))
        return fail(SWA_E_INVAL, "too many tokens: one head's key region must stay below 2 GiB");
    if (sws == 0 || sws < -1 || nfpb < 1 || S < 0) return fail(SWA_E_INVAL, "bad window arguments");
    const size_t need = swa_prefill_workspace_bytes(F, P, H, D, dtype);
    if (ws == nullptr || ws_bytes < need) return fail(SWA_E_INVAL, "workspace smaller than swa_prefill_workspace_bytes()");
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(SWA_E_INVAL, "workspace must be 256-byte aligned");
    const int W = sws == -1 ? -1 : sws * nfpb;
    const int rows = static_cast<int>(align_up(int64_t(F) * P + 64, 64));
    void* kreg = ws;
    void* vreg = static_cast<char*>(ws) + need / 2;
    // the F frames laid out as consecutive pages (frame f in rows [f*P, (f+1)*P))
    hipError_t e = swa::launch_append(dtype, H, D, F * P, 0, rows, k, v, kreg, vreg, nullptr, nullptr, nullptr, nullptr,
                                      nullptr, 0, swa::RetainArgs{0, 0, 0, nullptr, 0}, nullptr, stream);
    if (e != hipSuccess) return hip_fail(e, "chunk layout kernel launch");
    swa::AttnParams p{};
    p.q = q;
    p.kreg = kreg;
    p.vreg = vreg;
    p.out = out;
    p.lse = lse;
    p.nq = P;
    p.H = H;
    p.rs = int64_t(H) * D;
    p.hs = D;
    p.rows = rows;
    p.ncols = 1;
    p.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D)));
    p.F = F;
    p.W = W;
    p.S = S;
    p.fP = P;
    const int qrows = swa::attention_q_tile(dtype);
    p.qtiles = (P + qrows - 1) / qrows;
    e = swa::launch_attention(dtype, D, true, p, F * H * p.qtiles, stream);
    if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
    return SWA_OK;
}

int swa_prefill_mask(int F, int P, int sws, int nfpb, int S, int token_level, uint8_t* dev_out,
                     swa_stream_t stream) {
    if (dev_out == nullptr) return fail(SWA_E_INVAL, "null output");
    if (F < 1 || P < 1 || sws == 0 || sws < -1 || nfpb < 1 || S < 0) return fail(SWA_E_INVAL, "bad arguments");
    const int W = sws == -1 ? -1 : sws * nfpb;
    hipError_t e = swa::launch_mask(F, P, W, S, token_level ? 1 : 0, dev_out, stream);
    if (e != hipSuccess) return hip_fail(e, "mask kernel launch");
    return SWA_OK;
}

int swa_graph_create(swa_cache* c, void* const* q, const void* const* k, const void* const* v, void* const* out,
                     float* const* lse, const int32_t* pos, const float* const* qk_norm_weights, float eps,
                     swa_graph** g) {
    if (g == nullptr) return fail(SWA_E_INVAL, "null output handle");
    *g = nullptr;
    if (c == nullptr) return fail(SWA_E_INVAL, "null cache");
    if (c->dry) return fail(SWA_E_STATE, "bookkeeping-only cache cannot capture a step");
    if (c->cfg.dtype != SWA_BF16) return fail(SWA_E_UNSUPPORTED, "captured steps need a bf16 cache");
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return fail(SWA_E_INVAL, "null tensor array");
    const int nl = c->cfg.num_layers;
    for (int l = 0; l < nl; ++l) {
        if (q[l] == nullptr || k[l] == nullptr || v[l] == nullptr || out[l] == nullptr)
            return fail(SWA_E_INVAL, "null tensor");
        if (qk_norm_weights != nullptr && qk_norm_weights[l] == nullptr) return fail(SWA_E_INVAL, "null norm weights");
    }
    if (qk_norm_weights != nullptr && !(eps >= 0.f)) return fail(SWA_E_INVAL, "norm epsilon must be >= 0");
    if (pos != nullptr && c->cfg.rope_pairs_t + c->cfg.rope_pairs_h + c->cfg.rope_pairs_w == 0)
        return fail(SWA_E_INVAL, "positions given but the config has no rope bands");
    // one plan serves every layer: their rings must be in the same state
    const swa::RingCounters c0 = c->rings[0].counters();
    if (c0.pending) return fail(SWA_E_STATE, "a non-keyframe is pending");
    std::vector<swa::PageRec> p0, pl;
    c->rings[0].pages(&p0);
    for (int l = 1; l < nl; ++l) {
        c->rings[l].pages(&pl);
        const swa::RingCounters cl = c->rings[l].counters();
        bool same = cl.n_key == c0.n_key && cl.n_win == c0.n_win && cl.n_special == c0.n_special &&
                    pl.size() == p0.size();
        for (size_t i = 0; same && i < pl.size(); ++i)
            same = pl[i].frame == p0[i].frame && pl[i].slot == p0[i].slot && pl[i].row0 == p0[i].row0 &&
                   pl[i].nrows == p0[i].nrows && pl[i].region == p0[i].region;
        if (!same) return fail(SWA_E_STATE, "layers are in different ring states");
    }

    swa_graph* gr = new (std::nothrow) swa_graph();
    if (gr == nullptr) return fail(SWA_E_INVAL, "out of host memory");
    gr->c = c;
    hipStream_t s = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e != hipSuccess) {
        delete gr;
        return hip_fail(e, "capture stream");
    }
    e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    int rc = e == hipSuccess ? SWA_OK : hip_fail(e, "begin capture");
    for (int l = 0; rc == SWA_OK && l < nl; ++l) {
        swa::NormArgs norm{qk_norm_weights != nullptr ? qk_norm_weights[l] : nullptr, eps};
        rc = enqueue_planned_layer(c, l, q[l], k[l], v[l], pos, qk_norm_weights != nullptr ? &norm : nullptr,
                                   out[l], lse != nullptr ? lse[l] : nullptr, s);
    }
    if (e == hipSuccess) {
        const hipError_t e2 = hipStreamEndCapture(s, &gr->graph);
        if (rc == SWA_OK && e2 != hipSuccess) rc = hip_fail(e2, "end capture");
    }
    if (rc == SWA_OK) {
        e = hipGraphInstantiate(&gr->exec, gr->graph, nullptr, nullptr, 0);
        if (e != hipSuccess) rc = hip_fail(e, "graph instantiate");
    }
    (void)hipStreamDestroy(s);
    if (rc != SWA_OK) {
        delete gr;
        return rc;
    }
    *g = gr;
    return SWA_OK;
}

int swa_graph_step(swa_graph* g, int64_t t, int keyframe, swa_stream_t stream) {
    if (g == nullptr) return fail(SWA_E_INVAL, "null graph");
    swa_cache* c = g->c;
    const Layout& L = c->L;
    const int nl = c->cfg.num_layers;
    const swa::RingCounters c0 = c->rings[0].counters();
    for (int l = 1; l < nl; ++l) {
        const swa::RingCounters cl = c->rings[l].counters();
        if (cl.n_key != c0.n_key || cl.n_win != c0.n_win || cl.n_special != c0.n_special || cl.pending != c0.pending)
            return fail(SWA_E_STATE, "layers are in different ring states");
    }
    swa::AppendPlan plan;
    std::string err;
    int rc = c->rings[0].plan_append(t, keyframe != 0, &plan, &err);
    if (rc != SWA_OK) return fail(rc, err);
    // the ring as the attention sees it: after the append and, for a
    // keyframe, the eviction
    swa::Ring seen = c->rings[0];
    seen.commit_append(plan, t);
    if (keyframe) seen.evict();
    swa::StepPlan sp{};
    rc = fill_segs(seen, &sp.seg);
    if (rc != SWA_OK) return rc;
    sp.row0 = plan.slot * L.P;
    sp.append_meta = plan.keyframe ? plan.ord_index : static_cast<int32_t>(L.meta_pending);
    sp.frame = static_cast<int32_t>(t);
    sp.retain = plan.retain ? 1 : 0;
    if (plan.retain) {
        sp.retain_src = plan.victim_slot * L.P + c->cfg.special_row0;
        sp.retain_dst = L.special_row_base + plan.special_slot * L.ns;
        sp.retain_meta = static_cast<int32_t>(L.meta_special + plan.special_id_index);
        sp.victim_frame = static_cast<int32_t>(plan.victim_frame);
    }
    hipError_t e = swa::launch_plan_store(sp, c->step_plan(), stream);
    if (e != hipSuccess) return hip_fail(e, "step plan store");
    e = hipGraphLaunch(g->exec, stream);
    if (e != hipSuccess) return hip_fail(e, "graph launch");
    for (int l = 0; l < nl; ++l) {
        c->rings[l].commit_append(plan, t);
        if (keyframe) {
            c->rings[l].evict();
        } else {
            rc = c->rings[l].rollback(&err);
            if (rc != SWA_OK) return fail(rc, err);
        }
    }
    return SWA_OK;
}

int swa_graph_destroy(swa_graph* g) {
    delete g;
    return SWA_OK;
}

const char* swa_last_error(void) { return g_err.c_str(); }

}  // extern "C"

namespace swa {

int api_fail(int code, const char* msg) { return fail(code, msg); }

int64_t decode_partials_bytes(int G, int D, int max_cols) {
    const int64_t pieces = 2 * int64_t(max_cols);
    return align_up(pieces * G * D * 4, 256) + align_up(pieces * G * 2 * 4, 256);
}

int decode_step_impl(void* cache, size_t cache_bytes, int B, int Hq, int Hkv, int W, int D, int64_t pos,
                     const void* q, const void* k, const void* v, void* out, float* lse, void* part, int max_cols,
                     hipStream_t stream) {
    if (cache == nullptr || q == nullptr || k == nullptr || v == nullptr || out == nullptr)
        return fail(SWA_E_INVAL, "null pointer");
    if (B < 1 || Hkv < 1 || Hq < 1 || W < 1) return fail(SWA_E_INVAL, "B, Hq, Hkv and W must be >= 1");
    if (D != 32 && D != 64) return fail(SWA_E_UNSUPPORTED, "head_dim must be 32 or 64");
    if (Hq % Hkv != 0) return fail(SWA_E_INVAL, "Hq must be a multiple of Hkv");
    const int G = Hq / Hkv;
    if (G > attention_decode_q_rows()) return fail(SWA_E_UNSUPPORTED, "more than 32 query heads per kv head");
    if (pos < 0) return fail(SWA_E_INVAL, "position must be >= 0");
    if (int64_t(W) + 128 > (1ll << 30) || !row_space_fits(W, D, 2)) return fail(SWA_E_INVAL, "window too large");
    if (part == nullptr || max_cols < 1) return fail(SWA_E_INVAL, "no split-partial space");
    const DecodeLayout dl = decode_layout(B, Hkv, W, D);
    if (cache_bytes < static_cast<size_t>(dl.total)) return fail(SWA_E_INVAL, "cache smaller than swa_decode_cache_bytes()");
    if (reinterpret_cast<uintptr_t>(cache) % 256 != 0) return fail(SWA_E_INVAL, "cache must be 256-byte aligned");
    if (int64_t(B) * Hkv > (1 << 24)) return fail(SWA_E_INVAL, "too many sequences x kv heads");
    const int nh = B * Hkv;
    void* kreg = cache;
    void* vreg = static_cast<char*>(cache) + dl.k_bytes;
    const int slot = static_cast<int>(pos % W);

    const int n = static_cast<int>(std::min<int64_t>(pos + 1, W));   // live slots 0..n-1
    AttnParams p{};
    p.q = q;
    p.kreg = kreg;
    p.vreg = vreg;
    p.out = out;
    p.lse = lse;
    p.nq = G;
    p.H = nh;
    p.rs = D;
    p.hs = int64_t(G) * D;
    p.rows = static_cast<int>(dl.rows);
    p.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(D)));
    p.F = 1;
    p.seg.n = 1;
    for (int i = 0; i < kMaxSegs; ++i) {
        p.seg.lo[i] = p.seg.hi[i] = 0;
        p.seg.tile0[i] = 1 << 30;
    }
    p.seg.lo[0] = 0;
    p.seg.hi[0] = n;
    p.seg.tile0[0] = 0;
    const int tiles = tiles_of(0, n);
    p.seg.total_tiles = tiles;
    p.qtiles = 1;
    int64_t cols = std::min<int64_t>(decode_fit(D), max_cols);
    cols = std::max<int64_t>(1, std::min<int64_t>(cols, int64_t(nh) * tiles));
    p.ncols = static_cast<int>(cols);
    const int64_t pieces = 2 * int64_t(max_cols);
    p.dk = k;                                   // the new token goes in with the attention launch
    p.dv = v;
    p.dslot = slot;
    p.part_o = static_cast<float*>(part);
    p.part_ml = reinterpret_cast<float*>(static_cast<char*>(part) + align_up(pieces * G * D * 4, 256));
    hipError_t e = launch_attention_decode(D, p, p.ncols, stream);
    if (e != hipSuccess) return hip_fail(e, "decode attention kernel launch");
    if (!(p.ncols <= nh && nh % p.ncols == 0)) {
        e = launch_merge(D, nh, G, tiles, p.ncols, p.part_o, p.part_ml, out, lse, p.rs, p.hs, nullptr, stream);
        if (e != hipSuccess) return hip_fail(e, "decode merge kernel launch");
    }
    return SWA_OK;
}

}  // namespace swa
