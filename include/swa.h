/*
 * swa.h -- C ABI of the MI355X (gfx950) frame-block sliding-window attention
 * library over a streaming, paged KV cache.
 *
 * Sources of the semantics (cited by page title and section):
 *  [G]  "Sliding Window Attention Mechanism in AggregatorStream:
 *       Implementation and Configuration Guide" (instagit.com): sections
 *       "Mask Generation in CausalAttention", "KV Cache Eviction Strategy",
 *       "Manual Sliding-Window Mask Construction", "Cache Reset Between
 *       Sequences", FAQ.
 *  [IO] "Stream.py Aggregator Input and Output Formats: A Complete Technical
 *       Guide" (instagit.com): "Input Tensor Specifications", "Positional
 *       Embeddings" (3-D RoPE).
 *  [EX] the sliding-window-attention explainer (akshathtiwari.co.in): the
 *       rolling buffer written at slot i modulo W.
 *  [FB] codehub.bot symbol page of FlashInferBlock.forward: the streaming
 *       branch (keyframe: append_frame, evict_frames, compute_attention;
 *       non-keyframe: append with eviction deferred, compute_attention,
 *       rollback_last_frame).
 *
 * Conventions for every entry point:
 *  - Return 0 (SWA_OK) or a negative SWA_E_* code; nothing is thrown across
 *    the ABI.  swa_last_error() gives a thread-local message for the last
 *    failure on the calling thread.
 *  - Device pointers are caller-owned and must stay valid until the work
 *    enqueued on `stream` has finished.  Host pointers are read or written
 *    before the call returns.
 *  - Token tensors are contiguous NHD: [tokens, H, D] with D fastest, in the
 *    element type named by `dtype` (SWA_BF16 = bfloat16, SWA_F32 = float).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream).  Ring bookkeeping is done on the host at enqueue time, so
 *    state errors are reported without reading the device.
 *  - A cache handle is not thread-safe.  Batch size is 1 per call.
 *  - No entry point allocates device memory (swa_graph_create aside: the
 *    HIP runtime allocates its own resources for a captured graph).
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t* swa_stream_t;

enum swa_status {
    SWA_OK = 0,
    SWA_E_INVAL = -1,        /* bad argument or config                        */
    SWA_E_STATE = -2,        /* call not allowed in the cache's current state */
    SWA_E_CAPACITY = -3,     /* window off and max_frames keyframes cached    */
    SWA_E_UNSUPPORTED = -4,  /* valid but not implemented (e.g. head_dim 48)  */
    SWA_E_HIP = -5           /* a HIP runtime call or launch failed           */
};

enum swa_dtype { SWA_BF16 = 0, SWA_F32 = 1 };

enum swa_region { SWA_REGION_FRAME = 0, SWA_REGION_SPECIAL = 1 };

/*
 * Cache configuration ([G] constructor arguments; [FB] evict_frames
 * arguments).
 *   tokens_per_frame P     patch + special tokens per frame ([IO]).
 *   head_dim D             32 or 64.
 *   sliding_window_size    in blocks; -1 switches the window off ([G] FAQ);
 *                          0 and values below -1 are rejected.
 *   num_frame_per_block    window length in frames is
 *                          W = sliding_window_size * num_frame_per_block
 *                          ([G] "Mask Generation in CausalAttention").
 *   scale_frames S         the first S keyframes are never evicted ([G]
 *                          "KV Cache Eviction Strategy").  S = 0 is the
 *                          include_scale_frames = false case.
 *   cross_frame_special    keep `special_rows` rows (starting at row
 *                          `special_row0` of each frame) of every evicted
 *                          frame ([G] eviction section and FAQ), for at most
 *                          `max_special_frames` (R) evicted frames, oldest
 *                          dropped first.  camera_only is special_rows = 1.
 *   max_frames             capacity in keyframes when the window is off.
 *   rope_pairs_t/h/w, rope_theta
 *                          3-D RoPE bands used by swa_stream_step when a
 *                          position array is given ([IO] "Positional
 *                          Embeddings"); pairs must add up to D/2.
 * Size limit: one head's K (and V^T) region, rows x D x element bytes with
 * rows = (page slots x P + R x special_rows) rounded up to 64 plus 64, must
 * stay below 2 GiB (the kernels address it with 32-bit offsets); larger
 * configs are rejected with SWA_E_INVAL.
 */
typedef struct swa_config {
    int32_t num_layers;
    int32_t tokens_per_frame;
    int32_t num_heads;
    int32_t head_dim;
    int32_t dtype;
    int32_t sliding_window_size;
    int32_t num_frame_per_block;
    int32_t scale_frames;
    int32_t cross_frame_special;
    int32_t special_row0;
    int32_t special_rows;
    int32_t max_special_frames;
    int32_t max_frames;
    int32_t rope_pairs_t;
    int32_t rope_pairs_h;
    int32_t rope_pairs_w;
    float rope_theta;
} swa_config;

/*
 * One record of a visible-page list, in key order: scale frames, retained
 * special rows (oldest evicted frame first), window frames, then a pending
 * non-keyframe.  region SWA_REGION_FRAME: `slot` is the page slot, row0 = 0,
 * nrows = P.  region SWA_REGION_SPECIAL: `slot` is the special-ring entry
 * (push index mod R), row0 = slot * special_rows, nrows = special_rows.
 */
typedef struct swa_page {
    int32_t frame;
    int32_t region;
    int32_t slot;
    int32_t row0;
    int32_t nrows;
} swa_page;

/*
 * Where the cache keeps its rows inside the caller's pool (bytes from the
 * pool base).  Per layer l, with E = element size:
 *   K   at k_offset + l*layer_bytes, laid out [H][rows][D]
 *   V^T at v_offset + l*layer_bytes, laid out [H][rows/64][D][64]: blocks
 *       of 64 key positions, each a [D][64] matrix (rows is a multiple of
 *       64), where key r is stored at position r with bits 2 and 3 swapped
 *       (a permutation inside every aligned group of 16 keys; it matches the
 *       key order of one MFMA lane's operand).  Element (h, d, position s)
 *       is at ((h * rows/64 + s/64) * D + d) * 64 + s % 64.
 * Page slot s holds a frame in rows [s*P, (s+1)*P); special-ring entry e
 * holds its rows at special_row_base + e*special_rows.
 * The work area [work_offset, work_offset + work_bytes) holds the partial
 * results of streaming attention calls and the step plan of captured steps;
 * it is scratch between calls.
 */
typedef struct swa_layout {
    int64_t layer_bytes;
    int64_t k_offset;
    int64_t v_offset;
    int64_t meta_offset;
    int64_t work_offset;
    int64_t work_bytes;
    int32_t rows;
    int32_t num_slots;
    int32_t special_row_base;
    int32_t elem_bytes;
    int32_t window_frames;    /* -1 when the window is off */
    int32_t scratch_slot;
} swa_layout;

typedef struct swa_cache swa_cache;

/* Bytes of device memory a cache with this config needs (0 if invalid). */
size_t swa_cache_pool_bytes(const swa_config* cfg);

/*
 * Create a cache over a caller-owned device pool of at least
 * swa_cache_pool_bytes(cfg) bytes (256-byte aligned).  The library keeps its
 * bookkeeping on the host and allocates no device memory; the pool's
 * contents need no initialisation.  dev_pool = NULL with pool_bytes = 0 makes a
 * bookkeeping-only cache: append/evict/rollback/reset and
 * kvcache_visible_pages work and enqueue nothing; every call that would touch
 * the device returns SWA_E_STATE.
 */
int swa_cache_create(const swa_config* cfg, void* dev_pool, size_t pool_bytes, swa_cache** out);
int swa_cache_destroy(swa_cache* cache);
int swa_cache_layout(const swa_cache* cache, swa_layout* out);

/*
 * Work split of the streaming bf16 attention.  0 (default): the
 * num_heads * n (head, key tile) space is cut into as many equal columns as
 * the GPU runs at once (one launch round, every work-group the same number
 * of tiles); pieces of heads cut by a column edge are merged by a second
 * kernel.  k >= 1: each head's key tiles are cut into k equal pieces
 * (k = 1: no partials, no merge); num_heads * k is capped at 256.
 * SWA_E_INVAL for k outside 0..256.
 */
int swa_cache_set_splits(swa_cache* cache, int splits);

/* Forget every cached frame of every layer ([G] "Cache Reset Between
 * Sequences": clean_kv_cache).  Host bookkeeping only; nothing enqueued. */
int kvcache_reset(swa_cache* cache, swa_stream_t stream);

/*
 * append_frame ([FB]).  k, v: device [P, H, D].  frame_t must exceed every
 * frame index appended to this layer since the last reset.
 * keyframe != 0: the frame takes keyframe ordinal n; slot n if n < S, else
 *   S + ((n - S) mod W) -- the rolling buffer of [EX], shifted past the
 *   scale slots.  When the window is full this overwrites the slot of the
 *   frame the following kvcache_evict drops; with cross_frame_special that
 *   frame's special rows are copied to the special ring first.
 *   SWA_E_STATE if an eviction is pending or a non-keyframe is pending.
 * keyframe == 0: the frame goes to the scratch slot with eviction deferred;
 *   it must be removed with kvcache_rollback before the next append.
 * With the window off: SWA_E_CAPACITY once max_frames keyframes are cached.
 */
int kvcache_append(swa_cache* cache, int layer, int64_t frame_t, const void* k, const void* v,
                   int keyframe, swa_stream_t stream);

/* evict_frames ([FB]; rule of [G] "KV Cache Eviction Strategy"): when more
 * than W + S keyframes are cached, drop cached positions [S, n_cached - W).
 * No-op with the window off or while a non-keyframe is pending (eviction
 * deferred).  Host bookkeeping only. */
int kvcache_evict(swa_cache* cache, int layer, swa_stream_t stream);

/* rollback_last_frame ([FB]): drop the pending non-keyframe.  SWA_E_STATE if
 * there is none.  Host bookkeeping only. */
int kvcache_rollback(swa_cache* cache, int layer, swa_stream_t stream);

/* compute_attention ([FB]): attention of q (device [P, H, D]) over every
 * visible row of the layer -- scale frames, retained special rows, window
 * frames and a pending non-keyframe -- with softmax scale 1/sqrt(D).  Writes
 * out (device [P, H, D]) and, if not NULL, lse (device float [H, P]).
 * SWA_E_STATE if nothing is cached, or if a keyframe append has filled the
 * window past W frames and kvcache_evict has not run yet: [G] "KV Cache
 * Eviction Strategy" evicts before attention, and the append has already
 * overwritten the page of the frame that eviction drops. */
int kvcache_attend(swa_cache* cache, int layer, const void* q, void* out, float* lse, swa_stream_t stream);

/* Host copy of the layer's visible-page list (records in key order).  Writes
 * min(n, cap) records to `out` and the full count to *n_out.  Between a
 * keyframe append into a full window and its kvcache_evict the list still
 * names the frame the eviction will drop, although its page already holds
 * the new frame (bookkeeping view; kvcache_attend refuses that state). */
int kvcache_visible_pages(const swa_cache* cache, int layer, swa_page* out, int cap, int* n_out);

/* The same list built on the device from the device-side frame tables (the
 * page-list builder kernel), copied back; synchronises `stream`.  A test
 * export: the attention kernels take their key rows from the host ring, not
 * from this list.  SWA_E_STATE while an eviction is pending (see
 * kvcache_attend) and on a bookkeeping-only cache. */
int kvcache_read_device_pages(swa_cache* cache, int layer, swa_page* host_out, int cap, int* n_out,
                              swa_stream_t stream);

/*
 * 3-D RoPE in place on q and k, device [n_tokens, H, D] ([IO] "Positional
 * Embeddings": head_dim/2 complex values).  Pair p = (x[2p], x[2p+1]).
 * Pairs [0, pairs_t) use pos_thw[n*3+0], the next pairs_h use [n*3+1], the
 * last pairs_w use [n*3+2]; local pair kk of a band with d_b pairs turns by
 * pos * theta^(-kk/d_b) radians.  pos_thw: device int32 [n_tokens, 3].
 * Either q or k may be NULL.
 */
int rope3d_apply(void* q, void* k, const int32_t* pos_thw, int n_tokens, int H, int D, int pairs_t,
                 int pairs_h, int pairs_w, float theta, int dtype, swa_stream_t stream);

/*
 * One streaming step of one layer ([FB] streaming branch).
 * keyframe:     [rope] -> append -> evict -> attend.
 * non-keyframe: [rope] -> append (eviction deferred) -> attend -> rollback.
 * q: device [P, H, D]; rotated in place when pos_thw is not NULL.
 * k, v: device [P, H, D]; not modified (the rotated k goes to the cache).
 * pos_thw: device int32 [P, 3] or NULL (no RoPE).
 * out: device [P, H, D] (dtype of the cache); lse: device float [H, P]
 * (natural log of each row's softmax denominator, scores scaled by
 * 1/sqrt(D)) or NULL.
 */
int swa_stream_step(swa_cache* cache, int layer, int64_t frame_t, void* q, const void* k,
                    const void* v, const int32_t* pos_thw, int keyframe, void* out, float* lse,
                    swa_stream_t stream);

/*
 * Per-head layer norm of q and k in place, device [n_tokens, H, D].  The
 * streaming branch's pre-attention pass ([FB]) applies a q norm and a k norm
 * after the reshape to heads and before RoPE; their kind is not stated there
 * and is read as a layer norm over head_dim: each (token, head) row minus
 * its mean, divided by sqrt(biased variance + eps), times weight[d] plus
 * bias[d].  weights: device float [4][D] = q weight, q bias, k weight,
 * k bias (shared by all heads).  Math in float, one rounding to dtype.
 * Either q or k may be NULL.  SWA_E_INVAL for null weights, eps < 0 or a
 * bad shape; SWA_E_UNSUPPORTED for head_dim other than 32 or 64.
 */
int qk_norm_apply(void* q, void* k, int n_tokens, int H, int D, const float* weights, float eps, int dtype,
                  swa_stream_t stream);

/*
 * swa_stream_step with the q/k norm fused into the append pass ([FB]: the
 * pre-attention pass normalises q and k, then applies RoPE, then the frame
 * is appended): q is normalised (and rotated when pos_thw is not NULL) in
 * place; k is normalised (and rotated) on its way into the cache; v is
 * copied.  weights and eps as in qk_norm_apply.  Same errors as
 * swa_stream_step, plus SWA_E_INVAL for null weights or eps < 0.
 */
int swa_stream_step_normed(swa_cache* cache, int layer, int64_t frame_t, void* q, const void* k, const void* v,
                           const float* qk_norm_weights, float eps, const int32_t* pos_thw, int keyframe,
                           void* out, float* lse, swa_stream_t stream);

/*
 * One streaming step of every layer as one captured HIP graph.  The
 * streaming branch of [FB] runs, per layer, the pre-attention pass as one
 * captured graph and then append, evict and attention; here the whole step
 * of all num_layers layers is captured once and replayed for every frame.
 * Every value that changes from frame to frame -- the append destination,
 * the displaced frame's special-row copy, the frame id and the visible key
 * segments -- is read by the kernels from a step plan in device memory (in
 * the cache's work area), which swa_graph_step stores before each replay.
 *
 * swa_graph_create: bf16 caches only.  q, k, v, out: host arrays of
 *   num_layers device pointers, each [P, H, D], fixed for the graph's
 *   lifetime (the caller writes each frame's q, k, v there before its step;
 *   q is normalised and rotated in place as in swa_stream_step_normed).
 *   lse: NULL, or a host array of num_layers device float [H, P] pointers
 *   (entries may be NULL).  pos: NULL (no RoPE) or one device int32 [P, 3]
 *   buffer shared by the layers, rewritten by the caller per frame.
 *   qk_norm_weights: NULL (no norm) or a host array of num_layers device
 *   float [4][D] pointers; eps as in qk_norm_apply.  Every layer must be in
 *   the same ring state with no non-keyframe pending.  The work split in
 *   force (swa_cache_set_splits) is fixed into the graph.  Capturing and
 *   instantiating the graph lets the HIP runtime allocate its own
 *   resources; swa_graph_step allocates nothing.
 *   Errors: SWA_E_INVAL (null pointers, eps < 0, positions without rope
 *   bands), SWA_E_STATE (bookkeeping-only cache, layers in different
 *   states, a pending non-keyframe), SWA_E_UNSUPPORTED (F32 cache),
 *   SWA_E_HIP.
 * swa_graph_step: the step of frame_t for every layer, with the semantics
 *   of swa_stream_step (keyframe: append, evict, attend; non-keyframe:
 *   append with eviction deferred, attend, roll back).  Enqueues one small
 *   plan-store kernel and the graph on `stream`.  Steps of one cache must
 *   be ordered on one stream (the plan is shared).  The host ring
 *   bookkeeping of every layer advances as with per-layer calls, so the
 *   per-layer entry points and page lists stay valid; after a per-layer
 *   call leaves the layers in different states, SWA_E_STATE.
 * swa_graph_destroy: releases the graph (not the cache, which must outlive
 *   it).
 */
typedef struct swa_graph swa_graph;
int swa_graph_create(swa_cache* cache, void* const* q, const void* const* k, const void* const* v,
                     void* const* out, float* const* lse, const int32_t* pos_thw,
                     const float* const* qk_norm_weights, float eps, swa_graph** graph);
int swa_graph_step(swa_graph* graph, int64_t frame_t, int keyframe, swa_stream_t stream);
int swa_graph_destroy(swa_graph* graph);

/*
 * Token-level decode over per-sequence rolling buffers ([EX]: the key and
 * value of the token at position i live in slot i mod W, a fixed W-slot
 * cache; each token attends itself and the W - 1 tokens before it).  With
 * grouped-query heads (the explainer pairs the window with grouped-query
 * attention), query head h reads kv head h / (Hq / Hkv).  bf16 only.
 *
 * cache: device buffer of swa_decode_cache_bytes(B, Hkv, W, D) bytes, 256-byte
 *   aligned, caller-owned: K [B*Hkv][rows][D] then V^T [B*Hkv][rows/64][D][64]
 *   (rows = W plus 64 rows of tile padding, rounded up to a multiple of 64;
 *   V^T blocks and key positions as in swa_layout).  Contents need no initialisation: slot s is read only
 *   after a step has written it.
 * swa_decode_step: all B sequences are at the same position pos (>= 0) and
 *   must have been stepped through positions 0 .. pos-1 before.  Writes
 *   k, v (device [B, Hkv, D]) into slot pos mod W, then attends q (device
 *   [B, Hq, D]) over the min(pos+1, W) live slots.  out: device [B, Hq, D];
 *   lse: device float [B, Hq] (natural log, scores scaled by 1/sqrt(D)) or
 *   NULL.  work: device scratch of swa_decode_workspace_bytes(Hq, Hkv, D)
 *   bytes, 256-byte aligned (split partials; contents need no
 *   initialisation, no state kept between calls).
 * Errors: SWA_E_INVAL for null pointers, sizes < 1, Hq not a multiple of
 *   Hkv, pos < 0, too small or misaligned buffers; SWA_E_UNSUPPORTED for
 *   head_dim other than 32 or 64 or more than 32 query heads per kv head.
 *   The size queries return 0 for invalid arguments, including windows
 *   whose rows x D x 2 bytes reach 2 GiB per buffer.
 */
size_t swa_decode_cache_bytes(int B, int Hkv, int W, int D);
size_t swa_decode_workspace_bytes(int Hq, int Hkv, int D);
int swa_decode_step(void* cache, size_t cache_bytes, int B, int Hq, int Hkv, int W, int D, int64_t pos,
                    const void* q, const void* k, const void* v, void* out, float* lse, void* work,
                    size_t work_bytes, swa_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): swa_decode_step
 * with its split partials in a static device array of
 * SWA_DECODE_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on each
 * GPU it runs on until the process ends, instead of a caller workspace.  Same
 * arguments, kernels, work split and results as swa_decode_step.  Allocates
 * nothing; the first call on a device looks up the array's device address.
 * Limit: (Hq / Hkv) * (head_dim + 2) <= 1024 (15 query heads per kv head at
 * head_dim 64, 30 at 32), else SWA_E_CAPACITY.  Every call on one GPU shares
 * its array: calls that overlap on one GPU (different streams, or threads)
 * race and must be serialised by the caller.
 */
#define SWA_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)
int swa_decode_step_noalloc(void* cache, size_t cache_bytes, int B, int Hq, int Hkv, int W, int D, int64_t pos,
                            const void* q, const void* k, const void* v, void* out, float* lse,
                            swa_stream_t stream);

/*
 * Masked prefill of F frames submitted at once ([G] "Mask Generation in
 * CausalAttention"): query frame i sees key frame j iff j <= i and
 * (j >= i - W + 1 or j < scale_frames), W = sliding_window_size *
 * num_frame_per_block (-1: no window).  q, k, v, out: device [F*P, H, D];
 * lse: device float [H, F*P] or NULL.  Both dtypes need a device workspace
 * of swa_prefill_workspace_bytes() bytes, 256-byte aligned (the frames' keys
 * and transposed values are laid out there as consecutive pages; contents
 * need no initialisation).  SWA_E_INVAL (and a size query of 0) when one
 * head's F*P key rows, rounded up to 64 plus 64, times D times the element
 * size reach 2 GiB.
 */
size_t swa_prefill_workspace_bytes(int F, int P, int H, int D, int dtype);
int swa_prefill_masked(const void* q, const void* k, const void* v, int F, int P, int H, int D,
                       int sliding_window_size, int num_frame_per_block, int scale_frames, int dtype,
                       void* out, float* lse, void* workspace, size_t workspace_bytes,
                       swa_stream_t stream);

/*
 * The prefill visibility as bytes (1 = visible) from the same device
 * predicate the prefill kernels use: [F, F] if token_level == 0, else
 * [F*P, F*P].  dev_out: device uint8.
 */
int swa_prefill_mask(int F, int P, int sliding_window_size, int num_frame_per_block,
                     int scale_frames, int token_level, uint8_t* dev_out, swa_stream_t stream);

/* Message for the last failing call on this thread ("" if none). */
const char* swa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
