/*
 * kvstream.h -- C ABI of the bounded streaming KV cache for one AMD Instinct
 * MI355X (gfx950): paged frame-to-cache attention plus the cache-management
 * step (page write, sliding-window eviction, CLCES scoring, top-k compaction)
 * and diversity-scored per-head pruning.
 *
 * The operations follow these pages:
 *   [GCT]  "How GCTStream Implements Streaming 3D Reconstruction with KV Cache"
 *          (instagit explainer of Robbyant/lingbot-map)
 *   [FPS]  "Can LingBot-Map Achieve 20 FPS Streaming 3D Reconstruction?"
 *          (instagit explainer of Robbyant/lingbot-map)
 *   [SCV]  "StreamCacheVGGT: ..." (CSDN article), section 2.1 (CLCES)
 *   [INF]  "InfiniteVGGT: Visual Geometry Grounded Transformer for Endless
 *          Streams" (howistudyai explainer)
 *
 * Conventions for every entry point:
 *   - Every function returns a kv_status; nothing throws across the ABI.
 *     On any error the pool's state is unchanged and kv_last_error() returns
 *     a message for the calling thread.
 *   - All buffers named *_dev are device memory owned by the caller (the
 *     library never allocates device memory).  Host pointers are named
 *     plainly.  "stream" is a hipStream_t passed as void* (NULL = the null
 *     stream); device work is enqueued on it and the call returns without
 *     waiting, except where a function says it synchronises.
 *   - Layouts are row-major.  A frame's K, V and Q are [n_tokens][H][D].
 *   - Calls on one pool must not overlap from several host threads.
 *   - The device work of every call on one pool uses the pool's workspace
 *     (page-table mirrors, attention partials, CLCES and diversity scratch):
 *     issue a pool's calls on one stream, or order the streams with events,
 *     so that no two of its calls run on the GPU at once.
 */
#ifndef KVSTREAM_H
#define KVSTREAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kv_pool kv_pool_t;

typedef enum {
  KV_OK = 0,
  KV_ERR_ARG = -1,      /* null pointer, bad layer, out-of-range parameter        */
  KV_ERR_SHAPE = -2,    /* n_tokens != page_tokens, n_q out of range, bad sizes   */
  KV_ERR_NO_PAGES = -3, /* the layer's page pool is exhausted                     */
  KV_ERR_STATE = -4,    /* call out of order (frame index, empty cache, no device) */
  KV_ERR_HIP = -5,      /* a HIP runtime call failed                              */
  KV_ERR_NAN = -6       /* a raw score is NaN or negative                         */
} kv_status;

typedef enum { KV_BF16 = 0, KV_FP32 = 1 } kv_dtype;

/* kv_append_frame flag: attend this frame once, never persist it ([GCT]
 * "Selective Frame Caching with Skip Append", _set_skip_append(True)). */
#define KV_TRANSIENT 1u

/* Pool configuration.  The defaults of the pages are sliding_window = 64
 * frames and scale_frames = 8 ([FPS] "Sliding-Window Eviction Strategy"). */
typedef struct {
  int32_t num_layers;        /* >= 1                                               */
  int32_t num_heads;         /* >= 1                                               */
  int32_t head_dim;          /* must be 64                                         */
  int32_t page_tokens;       /* tokens per frame = tokens per page, 1..8192        */
  int32_t dtype;             /* kv_dtype of K, V, Q and the output                 */
  int32_t scale_frames;      /* first frames never evicted nor scored (0 = none)   */
  int32_t sliding_window;    /* persisted non-scale frames kept (0 = no window)    */
  int32_t keyframe_interval; /* >= 1: frame t persists iff t < S or (t-S) % k == 0 */
  int32_t pages_per_layer;   /* page ids per layer, >= 1                           */
  int32_t max_queries;       /* largest n_q of stream_attend, >= 1                 */
  int32_t max_splits;        /* split-KV partitions of one attention call, 1..64   */
  int32_t max_window;        /* largest CLCES layer window, 1..8                   */
  int32_t special_tokens;    /* 0 = off; else the first special_tokens slots of    */
                             /* every frame survive its window eviction ([GCT]     */
                             /* "Special Token Persistence"), 0..page_tokens       */
} kv_pool_config;

/* score_and_compact flags: return once the step is enqueued; reuse the ranks
 * of window layers from earlier steps over the same candidates (see there);
 * rank by the multi-pass radix sort whatever the size (the library otherwise
 * picks the faster of its two rank methods by size; both give the same
 * ranks). */
#define KV_CLCES_DEFER 1u
#define KV_CLCES_REUSE_RANKS 2u
#define KV_CLCES_RANK_RADIX 4u

/* Parameters of one CLCES step ([SCV] 2.1.1-2.1.3): window W = 5 layers,
 * lambda = 0.5 on the pages; keep_count = tokens kept (the budget); flags =
 * a combination of KV_CLCES_DEFER, KV_CLCES_REUSE_RANKS and
 * KV_CLCES_RANK_RADIX; s_hat_out:
 * optional device float64 [N], the fused score of every candidate in
 * candidate order (NULL: not written). */
typedef struct {
  int32_t window;
  uint32_t flags;
  double lambda;
  int64_t keep_count;
  double* s_hat_out;
} kv_clces_params;

/* Cache statistics ([GCT] "Cache Monitoring", get_kv_cache_info()). */
typedef struct {
  int32_t persisted_frames; /* frames in the layer's table                        */
  int32_t pages_used;       /* = persisted_frames + special_pages                 */
  int32_t pages_free;
  int32_t transient_pending;/* 1 if a transient frame waits for stream_attend     */
  int64_t tokens;           /* sum of page lengths (a page's longest head)        */
  int64_t bytes;            /* device bytes of the used pages                     */
  int64_t evictions;        /* pages evicted by the window since the last reset   */
  int64_t compactions;      /* score_and_compact steps that dropped tokens        */
  int64_t last_keep_count;  /* tokens kept by the last such step                  */
  int64_t merges;           /* pages released by kv_merge_pages                   */
  int64_t prunes;           /* kv_diversity_prune steps that dropped tokens       */
  int64_t special_pages;    /* pages holding special tokens of evicted frames     */
  int64_t special_tokens;   /* special tokens held (included in tokens)           */
} kv_cache_info;

/* Device memory layout of the pool, for callers that read pages directly.
 * The pool holds num_layers * (pages_per_layer + 1) pages; page id p of layer
 * l starts at byte (l * (pages_per_layer + 1) + p) * page_bytes; page id
 * pages_per_layer of each layer is that layer's transient page.  Inside a
 * page, with E = element size, Ts = token_stride (page_tokens rounded up to
 * 64), H heads and D = 64:
 *   K   at k_offset: [H][Ts][D]  -- token rows of each head, in slot order
 *   V   at v_offset: [H][Ts][D]  -- the same layout as K
 *   ids at id_offset: int32 [Ts] -- global token id frame*page_tokens + slot
 * Slots >= the page's length hold no data of the cache.  After
 * kv_diversity_prune the heads of a pruned page hold different tokens and
 * different counts (kv_get_head_lengths): the id row then describes none of
 * them, and rows past a head's own length hold no data. */
typedef struct {
  int64_t page_bytes;
  int64_t k_offset, v_offset, id_offset;
  int32_t token_stride;
  int32_t elem_bytes;
} kv_pool_layout;

/* Sizes of the pool and workspace buffers that kv_pool_create needs. */
kv_status kv_pool_required_bytes(const kv_pool_config* cfg, size_t* pool_bytes,
                                 size_t* workspace_bytes);

kv_status kv_pool_get_layout(const kv_pool_config* cfg, kv_pool_layout* out);

/* Create a pool over caller-owned device buffers of at least the required
 * sizes (256-byte aligned).  With pool_dev == NULL and workspace_dev == NULL
 * the pool is metadata-only: append/evict/score bookkeeping runs on the host
 * but every call that would touch the device returns KV_ERR_STATE.
 * The caller keeps ownership of both buffers; they must outlive the pool. */
kv_status kv_pool_create(const kv_pool_config* cfg, void* pool_dev, size_t pool_bytes,
                         void* workspace_dev, size_t workspace_bytes, kv_pool_t** out);

/* Release the pool's host state.  Waits for the read-back of any deferred
 * score_and_compact first and frees the pinned memory and events such steps
 * used; the caller's device buffers are left untouched. */
kv_status kv_pool_destroy(kv_pool_t* pool);

/* Drop every cached frame of every layer and reset statistics and frame
 * order ([GCT] "Cache Initialization and Cleanup", clean_kv_cache()).
 * Host-only; device contents are left as they are.  The result of a pending
 * deferred score_and_compact is waited for and dropped. */
kv_status kv_reset(kv_pool_t* pool);

/* Write frame frame_idx of one layer into the cache ([FPS] "Page-Aligned
 * Tensor Layout", _write_patch_page; [GCT] "Frame-by-Frame Causal
 * Processing").  k_dev, v_dev: [n_tokens][H][D] of the pool's dtype,
 * n_tokens must equal page_tokens.  A keyframe (see kv_pool_config) gets the
 * lowest free page id of the layer, appended at the end of its table; any
 * other frame, or any frame with KV_TRANSIENT, goes to the layer's transient
 * page and is attended by the next stream_attend only.  frame_idx must
 * increase from call to call on a layer (KV_ERR_STATE otherwise, and also
 * when a transient frame is still pending).  KV_ERR_NO_PAGES if no page id
 * is free.  Asynchronous on stream. */
kv_status kv_append_frame(kv_pool_t* pool, int32_t layer, int64_t frame_idx, const void* k_dev,
                          const void* v_dev, int32_t n_tokens, uint32_t flags, void* stream);

/* The same page write for layers first_layer .. first_layer+n_layers-1 in one
 * launch: k_dev, v_dev are [n_layers][n_tokens][H][D] (layer-major, each layer's
 * frame as for kv_append_frame).  Every layer is checked first; on any error no
 * layer changes.  Asynchronous on stream. */
kv_status kv_append_frame_layers(kv_pool_t* pool, int32_t first_layer, int32_t n_layers, int64_t frame_idx,
                                 const void* k_dev, const void* v_dev, int32_t n_tokens, uint32_t flags,
                                 void* stream);

/* Sliding-window eviction ([GCT] "Sliding Window Eviction"; [FPS]
 * "Sliding-Window Eviction Strategy", _apply_kv_cache_eviction_causal):
 * while the layer holds more than sliding_window persisted non-scale frames,
 * release the oldest one (whole page).  Scale frames are never evicted.
 * With special_tokens > 0 ([GCT] "Special Token Persistence"), the first
 * special_tokens rows of the victim (K and V of every head, and their ids)
 * are first appended to the layer's last special page; a new special page
 * (lowest free id, taken while the victim still holds its own) opens when
 * they do not fit in page_tokens slots.  Special pages follow the scale
 * frames in the table, are attended like any page, and are never evicted,
 * scored, pruned or merged.  Without special tokens this is host metadata
 * only; with them the copies are enqueued on `stream`.  KV_ERR_NO_PAGES
 * (nothing changes) if a special page is needed and no id is free.
 * n_evicted may be NULL. */
kv_status kv_evict(kv_pool_t* pool, int32_t layer, int32_t* n_evicted, void* stream);

/* Frame-to-cache attention ([GCT] "Frame-by-Frame Causal Processing" and
 * "Scale-Frame Phase"): for each query row i and head h,
 *   out[i,h,:] = sum_j softmax_j(sm_scale * q[i,h,:] . k[j,h,:]) v[j,h,:]
 * over every token j of the layer's table in table order, plus the pending
 * transient frame (which is consumed); after kv_diversity_prune, over the
 * rows head h holds in each page.  No token mask: a frame sees all of
 * its own tokens and, in the scale phase, the other scale frames.
 * q_dev, out_dev: [n_q][H][D] in the pool's dtype, 1 <= n_q <= max_queries.
 * lse_dev: optional fp32 [n_q][H] = natural log of the softmax denominator
 * (with the max included).  KV_ERR_STATE if the layer holds no token.
 * Asynchronous on stream; bf16 inputs use MFMA with fp32 accumulation. */
kv_status stream_attend(kv_pool_t* pool, int32_t layer, const void* q_dev, int32_t n_q,
                        float sm_scale, void* out_dev, float* lse_dev, void* stream);

/* stream_attend for callers that cannot allocate device memory or grow any
 * buffer during the call (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments, checks, split
 * count, kernels and results, bit for bit, but the split-KV partials go to a
 * static 64 MiB device array of the library (one copy per GPU, held until
 * the process ends; its address is looked up once per device on the first
 * call there) instead of the pool's workspace.  Allocates nothing: no
 * hipMalloc, no host allocation.  KV_ERR_SHAPE (nothing enqueued) when the
 * partials of the chosen split count, splits * n_q * H * (D + 2) * 4 bytes
 * plus alignment, exceed 64 MiB (the 1004-query, 16-head, 8-split call
 * needs 33.9 MB; one split needs none).  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (two streams, two threads)
 * race and corrupt each other's results; serialise them. */
kv_status stream_attend_scratch(kv_pool_t* pool, int32_t layer, const void* q_dev, int32_t n_q,
                                float sm_scale, void* out_dev, float* lse_dev, void* stream);

/* Measurement support: the next max_calls stream_attend / stream_attend_scratch
 * / kv_append_attend calls record a HIP event pair on their stream right
 * before and right after their attention kernel (before the split-KV
 * combine), so the kernel's own duration can be read without a profiler.
 * Creates the 2 * max_calls events here (max_calls = 0: frees them, timing
 * off); calls beyond max_calls record nothing.  kv_attend_timing_read waits for
 * the recorded events and returns the sum of the kernel times (ms) and the
 * number of calls timed.  kv_pool_destroy frees the events. */
kv_status kv_attend_timing(kv_pool_t* pool, int32_t max_calls);
kv_status kv_attend_timing_read(kv_pool_t* pool, double* total_ms, int32_t* n_calls);

/* One frame's cache step in one call: kv_append_frame(layer, frame_idx, k_dev,
 * v_dev, n_tokens, flags), then kv_evict(layer), then stream_attend(layer,
 * q_dev, n_q, sm_scale, out_dev, lse_dev), with the same arguments, checks,
 * results and page contents as those three calls in that order ([FPS]
 * "Page-Aligned Tensor Layout"; [GCT] "Frame-by-Frame Causal Processing").
 * The page write and the upload of the attention's page table are one
 * launch.  (stream_attend alone passes a shared table of up to 192 entries
 * in the attention kernel's arguments and uploads only longer or per-head
 * tables, so the fused call saves a launch only for those.)  n_q may
 * exceed n_tokens (the scale phase: the queries of every scale frame with
 * the last one's append).  n_evicted may be NULL.  On any error nothing
 * changes.  Asynchronous on stream. */
kv_status kv_append_attend(kv_pool_t* pool, int32_t layer, int64_t frame_idx, const void* k_dev,
                           const void* v_dev, int32_t n_tokens, uint32_t flags, const void* q_dev,
                           int32_t n_q, float sm_scale, void* out_dev, float* lse_dev, int32_t* n_evicted,
                           void* stream);

/* One CLCES step on a layer ([SCV] 2.1.1-2.1.4; top-k keep and compaction as
 * in [SCV] section 1 and [INF] "Rolling Memory").  Candidates: the tokens of
 * the layer's table, scale-frame pages excluded, in table order (N of them).
 * If N <= keep_count nothing happens and *n_kept = N.  Otherwise, for the
 * window layers w = max(0, layer-W+1) .. layer:
 *   R_w   = stable ascending rank of the raw score of each candidate at layer w
 *   r_w   = R_w / (N-1);  mu, sigma = mean and population std. deviation of r
 *   Cons  = max(0, 1 - sigma*sqrt(12));  s_hat = s_layer * (1 + lambda*Cons)
 * (float64, fixed order, no fused multiply-add), keep the keep_count
 * candidates first in (s_hat descending, index ascending) order, and compact
 * each page in place: with n of its slots kept, kept slots below n stay and
 * the dropped slots below n take the kept slots at or past n (both in
 * ascending slot order), moving K, V and token ids; emptied pages are
 * released.  The order of tokens inside a page is not part of the method.
 * score_table_dev: fp32 [score_rows][num_layers], row = global token id.
 * keep_ids_out_dev: optional int32 [keep_count], kept global token ids in
 * candidate order (table order, then slot order before compaction).
 * ranks_out_dev: optional int32 [n_window][N], oldest window layer first.
 * The rank of every window layer is kept in the pool after the step (one
 * slot per layer of max_window slots, least recently used replaced).  With
 * KV_CLCES_REUSE_RANKS ([SCV] 2.1.4: the rank history of a frame is reused
 * across layers) a window layer ranked by an earlier synchronous step over
 * the same candidate sequence is not ranked again: the layer must never have
 * been compacted, merged or pruned since kv_reset (its pages then hold whole
 * frames, so its candidate frames name the sequence), the score table pointer
 * and score_rows must be the same, and the caller guarantees that the table's
 * entries of those layers have not changed since (a new frame's scores go to
 * new rows).  kv_reset forgets every kept rank; deferred steps do not add to
 * the history.
 * n_kept: optional host int64.  KV_ERR_STATE on a layer that
 * kv_diversity_prune has pruned (its heads hold different tokens), and on a
 * pool with special_tokens > 0 (compaction would move the special tokens out
 * of a frame's first slots).
 * KV_ERR_NAN if a score read is NaN or negative (state unchanged), KV_ERR_ARG
 * for a token id >= score_rows or a bad parameter.  Waits for the new page
 * lengths only: the step writes each page's length into pinned host memory
 * mapped into the device (allocated by the pool on first use) as soon as it
 * is known, and the call returns while the rows may still be moving; work
 * issued later on the same stream (or one ordered after it) sees them moved.
 * With flags = KV_CLCES_DEFER the call returns once the step and the
 * read-back of its page lengths (into pinned host memory the pool allocates
 * on first use) are enqueued, *n_kept = keep_count, and the layer's host table
 * is brought up to date by the next call that names the layer (or by
 * kv_sync), which waits for that read-back first.  An error the kernels find
 * (NaN score, token id out of range) is then returned by that next call, which
 * does nothing else; the step moved no row and the layer is as it was.  Calls
 * on other layers do not wait.  Later calls must be issued on the same stream
 * (or one ordered after it): steps of all layers share the workspace. */
kv_status score_and_compact(kv_pool_t* pool, int32_t layer, const float* score_table_dev,
                            int64_t score_rows, const kv_clces_params* params,
                            int32_t* keep_ids_out_dev, int32_t* ranks_out_dev, int64_t* n_kept,
                            void* stream);

/* Completes the deferred score_and_compact of a layer (layer = -1: of every
 * layer) and returns its error, if any (the first one for -1).  A no-op where
 * nothing is pending. */
kv_status kv_sync(kv_pool_t* pool, int32_t layer);

/* Page merge: defragments the ragged pages that compaction leaves in a
 * token-budget layer (no passage of the pages covers it; it keeps the number of
 * live pages near 2*tokens/page_tokens over unbounded streams instead of one
 * page per frame ever seen).  Walks the layer's table in order from its first
 * non-scale page: a page whose length fits after the page before it (lengths
 * summing to at most page_tokens) is appended to that page -- its K and V rows
 * of every head and its token ids go to the slots after the earlier page's
 * rows -- and its page id is released.  The token sequence in table order is
 * unchanged, so scores, keep sets and attention see the same tokens in the
 * same order.  Device work (one launch per 128 merges) is enqueued on
 * `stream`; no sync.  n_merged: optional host int32, pages released.
 * On a layer that kv_diversity_prune has pruned (heads holding different
 * rows) the rule is applied per head: a page is appended to the page before
 * it when every head's two lengths sum to at most page_tokens, each head's
 * rows going after the rows that head already holds (one launch per 16
 * merges at 16 heads; at most 320 heads, KV_ERR_ARG beyond).  Each head's
 * token sequence in table order is unchanged, so the diversity top-K (ties
 * by candidate index) and attention see the same tokens in the same order.
 * Token ids are not moved there (such a page's id row describes none of its
 * heads).  KV_ERR_STATE if sliding_window > 0 (window eviction removes whole
 * frames, so its pages must hold one frame each). */
kv_status kv_merge_pages(kv_pool_t* pool, int32_t layer, int32_t* n_merged, void* stream);

/* kv_merge_pages for layers first_layer .. first_layer+n_layers-1 in one call:
 * the moves of every layer share launches.  n_merged: optional host int32
 * [n_layers], pages released per layer.  Every layer is checked first; on
 * an error no layer changes. */
kv_status kv_merge_pages_layers(kv_pool_t* pool, int32_t first_layer, int32_t n_layers, int32_t* n_merged,
                                void* stream);

/* Diversity scores of a layer's candidates ([INF] "Building Blocks",
 * "Cosine Similarity", step-by-step recipe steps 2-4).  Candidates: per head,
 * the rows of every page past the scale frames (the anchor), in table order,
 * then slot order (N_h of them).  With k_hat = k / |k| (0 for a zero key) and
 * m_h the mean of head h's k_hat,
 *   score = -(k_hat . m_h) / |m_h|     (every score 0 when m_h = 0),
 * computed in float64 from the stored keys with fixed-order sums.
 * scores_dev: optional float64 [H][score_stride] (score_stride >= max N_h),
 * the scores in candidate order; entries past N_h untouched.
 * *mean_diversity (host, required): the mean of the float64 scores over
 * every head and candidate (0 with no candidate).  KV_ERR_NAN if a candidate
 * key is not finite.  Synchronises the stream. */
kv_status kv_diversity_score(kv_pool_t* pool, int32_t layer, double* scores_dev, int64_t score_stride,
                             double* mean_diversity, void* stream);

/* kv_diversity_score for layers first_layer .. first_layer+n_layers-1 with
 * one wait for all of them (no score output); mean_diversity: host double
 * [n_layers].  KV_ERR_NAN names the first layer with a key that is not
 * finite.  Each layer keeps its keys in its own workspace slot, so a
 * kv_diversity_prune(_layers) of a layer that has not changed since reuses
 * them instead of scoring again. */
kv_status kv_diversity_score_layers(kv_pool_t* pool, int32_t first_layer, int32_t n_layers,
                                    double* mean_diversity, void* stream);

/* Per-layer budgets ([INF] "Building Blocks", recipe step 5): with
 * p = softmax(mean_diversity / tau) over the n_layers layers,
 *   keep_per_head[l] = floor(floor(p_l * total_tokens) / heads).
 * Host arithmetic in float64 (exp of the values minus their maximum); no
 * device work.  KV_ERR_ARG for tau <= 0, a non-finite mean / tau, heads < 1,
 * or total_tokens outside 0 .. 2^53. */
kv_status kv_layer_budgets(const double* mean_diversity, int32_t n_layers, double tau,
                           int64_t total_tokens, int32_t heads, int64_t* keep_per_head);

/* Diversity prune ([INF] recipe step 6, "Rolling Memory"): scores the
 * candidates as kv_diversity_score does, keeps each head's keep_per_head
 * candidates first in (float64 score descending, candidate index ascending)
 * order, and compacts every page and head in
 * place with the rule of score_and_compact (kept slots below the head's new
 * count n stay, the dropped slots below n take the kept slots at or past n,
 * both ascending), moving the K and V rows of that head; the id row does not
 * move.  A page whose heads are all empty is released; the scale frames
 * (anchor) are never touched.  Heads with N_h <= keep_per_head keep
 * everything; if every head does, nothing happens.  Afterwards heads hold
 * different tokens: stream_attend follows each head's rows, and
 * score_and_compact and kv_merge_pages refuse the layer (KV_ERR_STATE).
 * KV_ERR_STATE on a pool with special_tokens > 0 (as for score_and_compact).
 * scores_dev / score_stride as for kv_diversity_score.  kept_per_head:
 * optional host int64 [H] = min(keep_per_head, N_h).  KV_ERR_NAN (state
 * unchanged) if a candidate key is not finite.  Synchronises the stream. */
kv_status kv_diversity_prune(kv_pool_t* pool, int32_t layer, int64_t keep_per_head, double* scores_dev,
                             int64_t score_stride, int64_t* kept_per_head, void* stream);

/* kv_diversity_prune for layers first_layer .. first_layer+n_layers-1 with
 * one wait for all of them (no score output): keep_per_head is host int64
 * [n_layers] (one budget per layer, e.g. from kv_layer_budgets);
 * kept_per_head, optional, host int64 [n_layers][H].  A layer not scored in
 * its current state is scored first; every layer is scored before any row
 * moves, so on KV_ERR_NAN no layer changes. */
kv_status kv_diversity_prune_layers(kv_pool_t* pool, int32_t first_layer, int32_t n_layers,
                                    const int64_t* keep_per_head, int64_t* kept_per_head, void* stream);

/* Per-head lengths of the layer's pages, int32 [entry][H] in table order, cap
 * entries at most; *n_out = table size.  Equal to the page length in every
 * head unless kv_diversity_prune has run.  lens may be NULL. */
kv_status kv_get_head_lengths(const kv_pool_t* pool, int32_t layer, int32_t* lens, int32_t cap, int32_t* n_out);

/* Statistics of a layer ([GCT] "Cache Monitoring"). */
kv_status kv_get_info(const kv_pool_t* pool, int32_t layer, kv_cache_info* out);

/* The layer's persisted table in logical order: page ids (layer-local),
 * lengths and frame indices, cap entries at most; *n_out = table size (may
 * exceed cap).  A special page reports -1 - f, f the first frame whose special
 * tokens it holds.  Any output pointer may be NULL. */
kv_status kv_get_page_table(const kv_pool_t* pool, int32_t layer, int32_t* page_ids,
                            int32_t* page_lens, int64_t* frame_ids, int32_t cap, int32_t* n_out);

/* Split-KV partitions of stream_attend: 0 = automatic (default), else the
 * number to use, capped by max_splits, the token tiles and the workspace. */
kv_status kv_set_attend_splits(kv_pool_t* pool, int32_t splits);

/* KV tiles of the bf16 attention: KV_TILING_AUTO (default: packed for a
 * diversity-pruned layer, whose heads hold their tokens in different pages,
 * where tiles per page would leave more than 3% of the tile slots empty;
 * else per page), KV_TILING_PAGE (64-token tiles within each page, a page's
 * last tile partial) or KV_TILING_PACKED (64-token tiles over each head's
 * token sequence, across page ends).  The tiling partitions
 * the same sum: results agree up to fp32 reassociation.  KV_ERR_ARG for
 * another value. */
#define KV_TILING_AUTO 0
#define KV_TILING_PAGE 1
#define KV_TILING_PACKED 2
kv_status kv_set_attend_tiling(kv_pool_t* pool, int32_t tiling);

/* Message of the last failed call on this thread ("" if none). */
const char* kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVSTREAM_H */
