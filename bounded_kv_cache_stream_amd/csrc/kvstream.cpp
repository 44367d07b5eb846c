// C-ABI runtime of the bounded streaming KV cache (see include/kvstream.h).
//
// Owns host metadata only: per-layer page tables and page-id pools
// (policy.h), the carve-up of the caller's workspace, and the launch of the
// HIP kernels on the caller's stream.  Never allocates device memory.

#include "kvstream.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <memory>
#include <new>
#include <set>
#include <string>
#include <vector>

#include "clces.h"
#include "diversity.h"
#include "kernels.h"
#include "policy.h"

namespace {

thread_local std::string g_err;

kv_status fail(kv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kv_status fail(kv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

kv_status ok() {
  g_err.clear();
  return KV_OK;
}

kv_status hip_fail(hipError_t e, const char* what) {
  return fail(KV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

struct Layout {
  kvs::PageGeom geom;
  int64_t layer_pages;  // pages per layer including the transient page
  int64_t table_cap;    // device page-table entries per layer
  size_t pool_bytes;
  // workspace regions (byte offsets); the CLCES and diversity steps share one
  // region (each waits for its own work before it returns)
  size_t tables, part_o, part_ml, hlens, dkeys, rank_cache, clces, div, ws_bytes;
  int64_t part_rows;  // capacity in (split x query) rows
  kvs::ClcesSizes cl;
  kvs::DivSizes dv;
};

kv_status validate(const kv_pool_config* c) {
  if (!c) return fail(KV_ERR_ARG, "config is NULL");
  if (c->num_layers < 1 || c->num_layers > 4096) return fail(KV_ERR_ARG, "num_layers %d out of range", c->num_layers);
  if (c->num_heads < 1 || c->num_heads > 1024) return fail(KV_ERR_ARG, "num_heads %d out of range", c->num_heads);
  if (c->head_dim != kvs::kHeadDim) return fail(KV_ERR_ARG, "head_dim must be 64 (got %d)", c->head_dim);
  if (c->page_tokens < 1 || c->page_tokens > 8192)
    return fail(KV_ERR_ARG, "page_tokens %d out of range 1..8192", c->page_tokens);
  if (c->dtype != KV_BF16 && c->dtype != KV_FP32) return fail(KV_ERR_ARG, "unknown dtype %d", c->dtype);
  if (c->scale_frames < 0 || c->sliding_window < 0) return fail(KV_ERR_ARG, "negative scale_frames/window");
  if (c->keyframe_interval < 1) return fail(KV_ERR_ARG, "keyframe_interval must be >= 1");
  if (c->pages_per_layer < 1) return fail(KV_ERR_ARG, "pages_per_layer must be >= 1");
  if ((int64_t)c->pages_per_layer * c->page_tokens > (int64_t)1 << 30)
    return fail(KV_ERR_ARG, "pages_per_layer * page_tokens too large");
  if (c->max_queries < 1) return fail(KV_ERR_ARG, "max_queries must be >= 1");
  if (c->max_splits < 1 || c->max_splits > 64) return fail(KV_ERR_ARG, "max_splits must be 1..64");
  if (c->max_window < 1 || c->max_window > 8) return fail(KV_ERR_ARG, "max_window must be 1..8");
  if (c->special_tokens < 0 || c->special_tokens > c->page_tokens)
    return fail(KV_ERR_ARG, "special_tokens %d out of 0..page_tokens", c->special_tokens);
  return KV_OK;
}

Layout make_layout(const kv_pool_config* c) {
  Layout L{};
  const int64_t E = c->dtype == KV_BF16 ? 2 : 4;
  const int64_t ts = (c->page_tokens + kvs::kTile - 1) / kvs::kTile * kvs::kTile;
  const int64_t H = c->num_heads, D = kvs::kHeadDim;
  L.geom.esize = (int32_t)E;
  L.geom.ts = (int32_t)ts;
  L.geom.heads = (int32_t)H;
  L.geom.k_off = 0;
  L.geom.v_off = H * ts * D * E;
  L.geom.id_off = 2 * H * ts * D * E;
  L.geom.page_bytes = (int64_t)align_up((size_t)(L.geom.id_off + ts * 4));
  L.layer_pages = (int64_t)c->pages_per_layer + 1;
  L.pool_bytes = (size_t)(L.layer_pages * c->num_layers * L.geom.page_bytes);

  size_t off = 0;
  L.tables = off;
  L.table_cap = (H + 1) * (L.layer_pages + 1);  // entries per layer: room for one table per head
  off = align_up(off + sizeof(kvs::DevEntry) * (size_t)(L.table_cap * c->num_layers));
  L.part_rows = (int64_t)c->max_splits * std::min(c->max_queries, c->page_tokens);
  L.part_o = off;
  off = align_up(off + (size_t)L.part_rows * H * D * 4);
  L.part_ml = off;
  off = align_up(off + (size_t)L.part_rows * H * 2 * 4);
  L.hlens = off;  // per-head lengths of every physical page, int32 [page][H]
  off = align_up(off + (size_t)(L.layer_pages * c->num_layers) * (size_t)H * 4);
  // diversity keys of every layer, uint32 [layer][H][2][pages_per_layer * page_tokens]
  // (the high and the low word of each 64-bit order key): 8 bytes per (token,
  // head) against the 256 of its K and V rows
  L.dkeys = off;
  off = align_up(off + (size_t)c->num_layers * (size_t)H * (size_t)c->pages_per_layer * (size_t)c->page_tokens * 8);
  // CLCES ranks kept for later steps: int32 [max_window][pages_per_layer * page_tokens]
  L.rank_cache = off;
  off = align_up(off + (size_t)c->max_window * (size_t)c->pages_per_layer * (size_t)c->page_tokens * 4);
  L.cl = kvs::clces_sizes((int64_t)c->pages_per_layer * c->page_tokens, c->pages_per_layer, c->max_window,
                          (int32_t)ts);
  L.dv = kvs::div_sizes((int64_t)c->pages_per_layer * c->page_tokens, c->pages_per_layer, (int32_t)H,
                        c->num_layers);
  L.clces = off;
  L.div = off;
  off = align_up(off + std::max(L.cl.total, L.dv.total));
  L.ws_bytes = off;
  return L;
}

}  // namespace

struct kv_pool {
  kv_pool_config cfg;
  Layout lay;
  char* pool = nullptr;
  char* ws = nullptr;
  bool meta_only = false;
  int32_t splits_override = 0;
  int32_t tiling = KV_TILING_AUTO;
  std::vector<kvs::LayerPolicy> layers;
  std::vector<int64_t> scored_gen;  // per layer: the table generation its diversity keys belong to (-1: none)
  std::vector<kvs::DevEntry> scratch;  // host staging for table uploads
  // pinned host memory of the diversity calls (allocated at the first one):
  // the staging block copied to the device, then the read-back area; staged
  // is recorded after each call's kernels, and the staging block is rewritten
  // only once it has completed
  hipEvent_t wait_ev = nullptr;  // wait_stream's marker
  char* div_pinned = nullptr;
  char* div_pinned_dev = nullptr;  // the same block as the device addresses it (mapped, coherent)
  size_t div_stage_bytes = 0;
  hipEvent_t div_staged = nullptr;
  // deferred score_and_compact steps (KV_CLCES_DEFER): per layer, whether one
  // is pending, the event after its read-back, its page count and keep count;
  // the read-backs land in pinned host memory, (pages_per_layer + 1) ints per
  // layer (the error flag, then the new page lengths)
  struct Pending {
    bool active = false;
    hipEvent_t done = nullptr;
    int32_t n_entries = 0;
    int64_t keep = 0;
  };
  std::vector<Pending> pending;
  int32_t* pinned = nullptr;
  // synchronous score_and_compact: one word per page in mapped, coherent
  // pinned memory (allocated at the first such step), written by the index
  // step with the call's sequence number and the page's new length
  uint64_t* slots = nullptr;
  unsigned long long* slots_dev = nullptr;
  uint32_t slot_seq = 0;
  // CLCES rank history: per slot of the rank-cache region, which score-table
  // column it ranks and over which candidate sequence (score table, its rows,
  // the candidate frames of a layer never compacted, merged or pruned)
  struct RankSlot {
    bool valid = false;
    int32_t column = -1;
    const float* table = nullptr;
    int64_t rows = 0;
    std::vector<int64_t> frames;
    uint64_t used = 0;  // last step that named it
  };
  std::vector<RankSlot> rank_slots;
  uint64_t rank_clock = 0;
  // kv_attend_timing: event pairs recorded around the attention kernel of the
  // next calls (used pairs first)
  std::vector<std::pair<hipEvent_t, hipEvent_t>> timing;
  size_t timing_used = 0;
};

namespace {

// Waits until the stream has run everything enqueued on it so far, for a
// call that reads results back.  It polls an event: a blocking wait can
// return tens of microseconds after the GPU is done.  After kPollUs of
// polling it blocks instead.
constexpr double kPollUs = 20000.0;

hipError_t wait_stream(kv_pool_t* p, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (!p->wait_ev) e = hipEventCreateWithFlags(&p->wait_ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(p->wait_ev, st);
  if (e != hipSuccess) return e;
  const auto t0 = std::chrono::steady_clock::now();
  while ((e = hipEventQuery(p->wait_ev)) == hipErrorNotReady)
    if (std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count() > kPollUs)
      return hipEventSynchronize(p->wait_ev);
  return e;
}

// Pinned read-back slots of score_and_compact, (pages_per_layer + 1) ints per
// layer: the error flag, then the new page lengths.
hipError_t clces_pinned(kv_pool_t* p) {
  return hipHostMalloc(reinterpret_cast<void**>(&p->pinned),
                       sizeof(int32_t) * (size_t)p->cfg.num_layers * ((size_t)p->cfg.pages_per_layer + 1),
                       hipHostMallocDefault);
}

// The page words of synchronous score_and_compact steps.
hipError_t clces_slots(kv_pool_t* p) {
  const size_t bytes = sizeof(uint64_t) * (size_t)p->cfg.pages_per_layer;
  hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&p->slots), bytes, hipHostMallocMapped | hipHostMallocCoherent);
  if (e != hipSuccess) {
    p->slots = nullptr;
    return e;
  }
  std::memset(p->slots, 0, bytes);
  e = hipHostGetDevicePointer(reinterpret_cast<void**>(&p->slots_dev), p->slots, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(p->slots);
    p->slots = nullptr;
  }
  return e;
}

// Waits until the index step of the current synchronous step has written the
// words of all n pages (the kernels that move the rows may still run; later
// work on the stream is ordered after them).  Polls the words for kPollUs,
// then waits for the stream; *complete tells whether every word arrived.
hipError_t wait_slots(kv_pool_t* p, hipStream_t st, int32_t n, bool* complete) {
  const volatile uint64_t* w = p->slots;
  const uint64_t seq = p->slot_seq;
  int32_t i = 0;
  const auto t0 = std::chrono::steady_clock::now();
  for (;;) {
    while (i < n && (w[i] >> 32) == seq) ++i;
    if (i == n) break;
    if (std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count() > kPollUs) {
      const hipError_t e = hipStreamSynchronize(st);
      if (e != hipSuccess) return e;
      while (i < n && (w[i] >> 32) == seq) ++i;
      break;
    }
  }
  std::atomic_thread_fence(std::memory_order_acquire);
  *complete = i == n;
  return hipSuccess;
}

// Completes the layer's deferred score_and_compact, if one is pending: waits
// for its read-back and applies the new page lengths to the host table, or
// returns the step's error (its kernels then moved no row, and the table stays
// as it was).
kv_status settle(kv_pool_t* p, int32_t layer) {
  auto& ps = p->pending[(size_t)layer];
  if (!ps.active) return KV_OK;
  ps.active = false;
  hipError_t e = hipEventSynchronize(ps.done);
  if (e != hipSuccess) return hip_fail(e, "deferred score_and_compact");
  const int32_t* rb = p->pinned + (size_t)layer * ((size_t)p->cfg.pages_per_layer + 1);
  if (rb[0] & kvs::kClcesErrNan)
    return fail(KV_ERR_NAN, "layer %d: a raw score of the deferred score_and_compact is NaN or negative (nothing "
                            "changed)", layer);
  if (rb[0] & kvs::kClcesErrRow)
    return fail(KV_ERR_ARG, "layer %d: a token id of the deferred score_and_compact is >= score_rows (nothing "
                            "changed)", layer);
  if (rb[0]) return fail(KV_ERR_HIP, "layer %d: deferred CLCES consistency check failed (flag %d)", layer, rb[0]);
  std::vector<int32_t> nl(rb + 1, rb + 1 + ps.n_entries);
  int64_t kept = 0;
  for (int32_t v : nl) kept += v;
  if (kept != ps.keep)
    return fail(KV_ERR_HIP, "layer %d: deferred step kept %lld tokens, expected %lld", layer, (long long)kept,
                (long long)ps.keep);
  p->layers[(size_t)layer].apply_compaction(nl, kept);
  return KV_OK;
}

// Waits for a pending read-back and drops its result (reset, destroy).
void discard_pending(kv_pool_t* p) {
  for (auto& ps : p->pending)
    if (ps.active) {
      (void)hipEventSynchronize(ps.done);
      ps.active = false;
    }
}

// Every entry point that names a layer checks it here, which also completes a
// deferred step of that layer first (the const getters included: a pool is
// never created const).
kv_status check_layer(const kv_pool_t* p, int32_t layer) {
  if (!p) return fail(KV_ERR_ARG, "pool is NULL");
  if (layer < 0 || layer >= p->cfg.num_layers) return fail(KV_ERR_ARG, "layer %d out of range", layer);
  return settle(const_cast<kv_pool_t*>(p), layer);
}

int64_t phys_page(const kv_pool_t* p, int32_t layer, int32_t page) {
  const int32_t id = page < 0 ? p->cfg.pages_per_layer : page;  // -1 = transient page
  return (int64_t)layer * p->lay.layer_pages + id;
}

kvs::DevEntry* dev_table(const kv_pool_t* p, int32_t layer) {
  return reinterpret_cast<kvs::DevEntry*>(p->ws + p->lay.tables) + (int64_t)layer * p->lay.table_cap;
}

int32_t* hlens_dev(const kv_pool_t* p) { return reinterpret_cast<int32_t*>(p->ws + p->lay.hlens); }

// The sum of the lengths of a layer's candidate pages (every page past the
// scale frames): at least any head's candidate count, since a page's length
// is the largest of its heads'.  The exact per-head counts come from the
// device (the tables kernel) with each call's read-back; head_counts()
// computes them on the host where a call needs them without a launch.
int64_t candidate_bound(const kv_pool_t* pool, int32_t layer) {
  const auto& L = pool->layers[(size_t)layer];
  int64_t n = 0;
  for (size_t i = L.first_candidate(); i < L.table.size(); ++i) n += L.table[i].len;
  return n;
}

// Each head's candidate count of a layer, on the host.
std::vector<int64_t> head_counts(const kv_pool_t* pool, int32_t layer) {
  const auto& L = pool->layers[(size_t)layer];
  const int32_t H = pool->cfg.num_heads;
  std::vector<int64_t> n((size_t)H, 0);
  for (size_t i = L.first_candidate(); i < L.table.size(); ++i) {
    const auto& e = L.table[i];
    for (int32_t h = 0; h < H; ++h) n[(size_t)h] += e.hlen.empty() ? e.len : e.hlen[(size_t)h];
  }
  return n;
}

kv_status check_layers(const kv_pool_t* p, int32_t first, int32_t n) {
  if (!p) return fail(KV_ERR_ARG, "pool is NULL");
  if (n < 1 || first < 0 || first + n > p->cfg.num_layers)
    return fail(KV_ERR_ARG, "layers %d..%d out of range", first, first + n - 1);
  for (int32_t l = first; l < first + n; ++l) {
    kv_status s = settle(const_cast<kv_pool_t*>(p), l);
    if (s != KV_OK) return s;
  }
  return KV_OK;
}

// One diversity call over a set of layers (slots in order) and its launch
// arguments; the parameters and candidate pages of each slot are written
// straight into the pinned staging block.
struct DivBatch {
  std::vector<int32_t> layer;  // slot -> layer
  kvs::DivCall call{};
};

// The pinned block of the diversity calls (mapped into the device's address
// space): staging for every layer, then the
// larger of the two read-backs (scoring: totals, flags and head counts; prune:
// flags, head counts, kept totals and every layer's new lengths).
hipError_t div_pinned(kv_pool_t* pool) {
  if (pool->div_pinned) return pool->div_staged ? hipEventSynchronize(pool->div_staged) : hipSuccess;
  const kvs::DivSizes& z = pool->lay.dv;
  const size_t stage = (kvs::div_staging_bytes(z, z.layers) + 255) / 256 * 256;
  const size_t rb_score = (z.hcount - z.totals) + sizeof(int32_t) * (size_t)z.layers * z.h_max;
  const size_t rb_prune = (z.new_len - z.flags) + sizeof(int32_t) * (size_t)z.layers * z.p_max * z.h_max;
  // mapped: the first kernel of a call reads the staging block itself;
  // coherent: it sees the host's writes made before the launch
  hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&pool->div_pinned), stage + std::max(rb_score, rb_prune),
                               hipHostMallocMapped | hipHostMallocCoherent);
  if (e != hipSuccess) {
    pool->div_pinned = nullptr;
    return e;
  }
  e = hipHostGetDevicePointer(reinterpret_cast<void**>(&pool->div_pinned_dev), pool->div_pinned, 0);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&pool->div_staged, hipEventDisableTiming);
  if (e != hipSuccess) {
    (void)hipHostFree(pool->div_pinned);
    pool->div_pinned = nullptr;
    pool->div_staged = nullptr;
    return e;
  }
  pool->div_stage_bytes = stage;
  return hipSuccess;
}

char* div_readback(kv_pool_t* pool) { return pool->div_pinned + pool->div_stage_bytes; }

// Call after div_pinned() succeeded: stages every slot (its parameters, then
// its candidate pages: phys, len, tile_start = per-head lengths in the
// device array) in the pinned block and fills the launch arguments.
DivBatch div_batch(kv_pool_t* pool, const std::vector<int32_t>& layers, const std::vector<int64_t>& n_ub,
                   const std::vector<int64_t>& keep, const std::vector<char>& rescore, bool prune, double* scores,
                   int64_t stride) {
  DivBatch b;
  const kvs::DivSizes& z = pool->lay.dv;
  const int n = (int)layers.size();
  b.layer = layers;
  char* staging = pool->div_pinned;
  kvs::DivCall& c = b.call;
  c.ws = pool->ws + pool->lay.div;
  c.sizes = z;
  c.pool = pool->pool;
  c.geom = pool->lay.geom;
  c.hlen_dev = hlens_dev(pool);
  c.keys_dev = reinterpret_cast<uint32_t*>(pool->ws + pool->lay.dkeys);
  c.staging = pool->div_pinned_dev;
  c.n = n;
  c.prune = prune;
  c.scores_out = scores;
  c.score_stride = stride;
  const int64_t per_layer = 2 * (int64_t)pool->cfg.num_heads * pool->cfg.pages_per_layer * pool->cfg.page_tokens;
  for (int i = 0; i < n; ++i) {
    const int32_t layer = layers[(size_t)i];
    const auto& T = pool->layers[(size_t)layer];
    kvs::DevEntry* out = kvs::div_staging_bases(z, staging, i);
    int32_t P = 0;
    for (size_t j = T.first_candidate(); j < T.table.size(); ++j) {
      const auto& e = T.table[j];
      out[P++] = kvs::DevEntry{(int32_t)phys_page(pool, layer, e.page), e.len, e.hlen.empty() ? 0 : 1, 0};
    }
    kvs::DivLayer& L = kvs::div_staging_layers(staging)[i];
    L.keys_off = (int64_t)layer * per_layer;
    L.N = n_ub[(size_t)i];
    L.keep = keep[(size_t)i];
    L.P = P;
    L.rescore = rescore[(size_t)i];
    L.layer = layer;
    L.pad = 0;
    c.max_P = std::max(c.max_P, L.P);
    c.max_N = std::max(c.max_N, L.N);
    c.any_rescore = c.any_rescore || L.rescore;
  }
  return b;
}

// Scores layers first .. first+n-1, one wait for all of them.
kv_status diversity_score_range(kv_pool_t* pool, int32_t first, int32_t n, double* scores_dev, int64_t stride,
                                double* means, hipStream_t st) {
  std::vector<int32_t> layers;
  std::vector<int64_t> n_ub;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t nu = candidate_bound(pool, first + i);
    means[i] = 0.0;
    if (nu > 0) {
      layers.push_back(first + i);
      n_ub.push_back(nu);
    }
  }
  if (layers.empty()) return ok();
  if (pool->meta_only) return fail(KV_ERR_STATE, "metadata-only pool has no device memory");
  if (scores_dev) {
    const std::vector<int64_t> nh = head_counts(pool, first);
    const int64_t n_max = *std::max_element(nh.begin(), nh.end());
    if (stride < n_max)
      return fail(KV_ERR_SHAPE, "score_stride %lld < %lld candidates of one head", (long long)stride,
                  (long long)n_max);
  }
  const size_t m = layers.size();
  hipError_t e = div_pinned(pool);
  if (e != hipSuccess) return hip_fail(e, "diversity staging");
  DivBatch b = div_batch(pool, layers, n_ub, std::vector<int64_t>(m, 0), std::vector<char>(m, 1), false, scores_dev,
                         stride);
  for (int32_t l : layers) pool->scored_gen[(size_t)l] = -1;
  e = kvs::enqueue_diversity(b.call, st);
  const hipError_t staged = hipEventRecord(pool->div_staged, st);  // also after a failed launch: the copy may be queued
  if (e == hipSuccess) e = staged;
  if (e != hipSuccess) return hip_fail(e, "diversity scoring launch");
  // one read-back: the float64 score sums, then (adjacent) the error flags and
  // each head's candidate count
  const kvs::DivSizes& z = pool->lay.dv;
  const size_t flags_at = z.flags - z.totals, counts_at = z.hcount - z.totals;
  const int32_t H = pool->cfg.num_heads;
  char* rb = div_readback(pool);
  e = hipMemcpyAsync(rb, kvs::div_totals(b.call), counts_at + sizeof(int32_t) * m * (size_t)H,
                     hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = wait_stream(pool, st);
  if (e != hipSuccess) return hip_fail(e, "diversity scoring");
  const double* sums = reinterpret_cast<const double*>(rb);
  const int32_t* flags = reinterpret_cast<const int32_t*>(rb + flags_at);
  const int32_t* counts = reinterpret_cast<const int32_t*>(rb + counts_at);
  for (size_t i = 0; i < m; ++i)
    if (flags[i] & kvs::kDivErrNan) return fail(KV_ERR_NAN, "layer %d: a candidate key is not finite", layers[i]);
  for (size_t i = 0; i < m; ++i) {
    const int32_t l = layers[i];
    int64_t n_total = 0;
    for (int32_t h = 0; h < H; ++h) n_total += counts[i * (size_t)H + (size_t)h];
    means[l - first] = n_total > 0 ? sums[i] / (double)n_total : 0.0;
    pool->scored_gen[(size_t)l] = pool->layers[(size_t)l].gen;
  }
  return ok();
}

// Prunes layers first .. first+n-1 to keep[i] candidates per head, one wait
// for all of them.  Layers whose keys are not from a scoring of their
// current state are scored in the same call, before any row moves, so a key
// that is not finite in any layer leaves every layer unchanged.
kv_status diversity_prune_range(kv_pool_t* pool, int32_t first, int32_t n, const int64_t* keep, double* scores_dev,
                                int64_t stride, int64_t* kept, hipStream_t st) {
  const int32_t H = pool->cfg.num_heads;
  for (int32_t i = 0; i < n; ++i)
    if (keep[i] < 0) return fail(KV_ERR_ARG, "keep_per_head[%d] must be >= 0", i);
  if (pool->cfg.special_tokens > 0)
    return fail(KV_ERR_STATE, "a prune would move the special tokens out of a frame's first slots "
                              "(special_tokens > 0)");
  // a layer whose sum of page lengths exceeds its keep goes to the device; one
  // whose heads all turn out to hold at most keep candidates comes back
  // unchanged and is not counted as pruned
  std::vector<int32_t> layers;
  std::vector<int64_t> n_ub;
  std::vector<int64_t> kp;
  std::vector<char> rescore;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t nu = candidate_bound(pool, first + i);
    if (nu > keep[i]) {
      const int32_t l = first + i;
      layers.push_back(l);
      n_ub.push_back(nu);
      kp.push_back(keep[i]);
      rescore.push_back(scores_dev || pool->scored_gen[(size_t)l] != pool->layers[(size_t)l].gen);
    } else if (kept) {
      const std::vector<int64_t> nh = head_counts(pool, first + i);
      for (int32_t h = 0; h < H; ++h) kept[(int64_t)i * H + h] = std::min(keep[i], nh[(size_t)h]);
    }
  }
  if (layers.empty()) return ok();
  if (pool->meta_only) return fail(KV_ERR_STATE, "metadata-only pool has no device memory");
  if (scores_dev) {
    const std::vector<int64_t> nh = head_counts(pool, first);
    const int64_t n_max = *std::max_element(nh.begin(), nh.end());
    if (stride < n_max)
      return fail(KV_ERR_SHAPE, "score_stride %lld < %lld candidates of one head", (long long)stride,
                  (long long)n_max);
  }
  const size_t m = layers.size();
  hipError_t e = div_pinned(pool);
  if (e != hipSuccess) return hip_fail(e, "diversity staging");
  DivBatch b = div_batch(pool, layers, n_ub, kp, rescore, true, scores_dev, stride);
  std::vector<int64_t> gen_before(m);
  for (size_t i = 0; i < m; ++i) {
    gen_before[i] = pool->scored_gen[(size_t)layers[i]];
    pool->scored_gen[(size_t)layers[i]] = -1;
  }
  e = kvs::enqueue_diversity(b.call, st);
  const hipError_t staged = hipEventRecord(pool->div_staged, st);  // also after a failed launch: the copy may be queued
  if (e == hipSuccess) e = staged;
  if (e != hipSuccess) return hip_fail(e, "diversity prune launch");
  // one read-back: the error flags, then (adjacent) each head's candidate
  // count, each head's kept total and every slot's new lengths [slot][max_P][H]
  const kvs::DivSizes& z = pool->lay.dv;
  const size_t counts_at = (z.hcount - z.flags) / sizeof(int32_t), kept_at = (z.kept - z.flags) / sizeof(int32_t);
  const size_t len_at = (z.new_len - z.flags) / sizeof(int32_t);
  const size_t per_slot = (size_t)b.call.max_P * (size_t)H;
  int32_t* rb = reinterpret_cast<int32_t*>(div_readback(pool));
  e = hipMemcpyAsync(rb, kvs::div_flags(b.call), sizeof(int32_t) * (len_at + m * per_slot), hipMemcpyDeviceToHost,
                     st);
  if (e == hipSuccess) e = wait_stream(pool, st);
  if (e != hipSuccess) return hip_fail(e, "diversity prune");
  const int32_t* flags = rb;
  auto counts = [&](size_t i) { return rb + counts_at + i * (size_t)H; };
  auto kept_dev = [&](size_t i) { return rb + kept_at + i * (size_t)H; };
  auto nl = [&](size_t i) { return rb + len_at + i * per_slot; };
  for (size_t i = 0; i < m; ++i)
    if (flags[i] & kvs::kDivErrNan)
      return fail(KV_ERR_NAN, "layer %d: a candidate key is not finite (no layer changed)", layers[i]);
  for (size_t i = 0; i < m; ++i) {
    if (flags[i]) return fail(KV_ERR_HIP, "layer %d: diversity prune consistency check failed (flag %d, pool "
                                          "state undefined)", layers[i], flags[i]);
    for (int32_t h = 0; h < H; ++h) {
      const int64_t want = std::min<int64_t>(kp[i], counts(i)[h]);
      if (kept_dev(i)[h] != want)
        return fail(KV_ERR_HIP, "layer %d head %d: kept %d candidates, expected %lld (pool state undefined)",
                    layers[i], h, kept_dev(i)[h], (long long)want);
    }
  }
  for (size_t i = 0; i < m; ++i) {
    const int32_t l = layers[i];
    const int32_t* c = counts(i);
    if (*std::max_element(c, c + H) > kp[i]) {
      pool->layers[(size_t)l].apply_head_compaction(nl(i), H);
    } else {
      pool->scored_gen[(size_t)l] = gen_before[i];  // nothing moved: the keys still describe the layer
      if (rescore[i]) pool->scored_gen[(size_t)l] = pool->layers[(size_t)l].gen;
    }
    if (kept)
      for (int32_t h = 0; h < H; ++h) kept[(int64_t)(l - first) * H + h] = std::min<int64_t>(kp[i], c[h]);
  }
  return ok();
}

}  // namespace

extern "C" {

kv_status kv_pool_required_bytes(const kv_pool_config* cfg, size_t* pool_bytes, size_t* workspace_bytes) {
  kv_status s = validate(cfg);
  if (s != KV_OK) return s;
  Layout L = make_layout(cfg);
  if (pool_bytes) *pool_bytes = L.pool_bytes;
  if (workspace_bytes) *workspace_bytes = L.ws_bytes;
  return ok();
}

kv_status kv_pool_get_layout(const kv_pool_config* cfg, kv_pool_layout* out) {
  kv_status s = validate(cfg);
  if (s != KV_OK) return s;
  if (!out) return fail(KV_ERR_ARG, "out is NULL");
  Layout L = make_layout(cfg);
  out->page_bytes = L.geom.page_bytes;
  out->k_offset = L.geom.k_off;
  out->v_offset = L.geom.v_off;
  out->id_offset = L.geom.id_off;
  out->token_stride = L.geom.ts;
  out->elem_bytes = L.geom.esize;
  return ok();
}

kv_status kv_pool_create(const kv_pool_config* cfg, void* pool_dev, size_t pool_bytes, void* workspace_dev,
                         size_t workspace_bytes, kv_pool_t** out) {
  kv_status s = validate(cfg);
  if (s != KV_OK) return s;
  if (!out) return fail(KV_ERR_ARG, "out is NULL");
  Layout L = make_layout(cfg);
  const bool meta = pool_dev == nullptr && workspace_dev == nullptr;
  if (!meta) {
    if (!pool_dev || !workspace_dev) return fail(KV_ERR_ARG, "pool and workspace must both be given or both NULL");
    if (pool_bytes < L.pool_bytes)
      return fail(KV_ERR_SHAPE, "pool buffer too small: %zu < %zu bytes", pool_bytes, L.pool_bytes);
    if (workspace_bytes < L.ws_bytes)
      return fail(KV_ERR_SHAPE, "workspace too small: %zu < %zu bytes", workspace_bytes, L.ws_bytes);
    if ((reinterpret_cast<uintptr_t>(pool_dev) | reinterpret_cast<uintptr_t>(workspace_dev)) % kAlign)
      return fail(KV_ERR_ARG, "pool and workspace must be 256-byte aligned");
  }
  kv_pool_t* p = new (std::nothrow) kv_pool_t();
  if (!p) return fail(KV_ERR_ARG, "out of host memory");
  p->cfg = *cfg;
  p->lay = L;
  p->pool = static_cast<char*>(pool_dev);
  p->ws = static_cast<char*>(workspace_dev);
  p->meta_only = meta;
  p->layers.resize((size_t)cfg->num_layers);
  p->scored_gen.assign((size_t)cfg->num_layers, -1);
  p->pending.resize((size_t)cfg->num_layers);
  p->rank_slots.resize((size_t)cfg->max_window);
  for (auto& l : p->layers)
    l.init(cfg->pages_per_layer, cfg->scale_frames, cfg->sliding_window, cfg->keyframe_interval, cfg->page_tokens,
           cfg->special_tokens);
  // every page id of a layer plus its transient page: table uploads never grow the staging vector
  p->scratch.reserve((size_t)cfg->pages_per_layer + 2);
  *out = p;
  return ok();
}

namespace {
void free_timing(kv_pool_t* pool) {
  for (auto& pr : pool->timing) {
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  pool->timing.clear();
  pool->timing_used = 0;
}
}  // namespace

kv_status kv_attend_timing(kv_pool_t* pool, int32_t max_calls) {
  if (!pool) return fail(KV_ERR_ARG, "pool is NULL");
  if (max_calls < 0 || max_calls > (1 << 20)) return fail(KV_ERR_ARG, "max_calls %d out of 0..2^20", max_calls);
  free_timing(pool);
  for (int32_t i = 0; i < max_calls; ++i) {
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    if (e != hipSuccess) {
      if (a) (void)hipEventDestroy(a);
      free_timing(pool);
      return hip_fail(e, "timing events");
    }
    pool->timing.emplace_back(a, b);
  }
  return ok();
}

kv_status kv_attend_timing_read(kv_pool_t* pool, double* total_ms, int32_t* n_calls) {
  if (!pool || !total_ms || !n_calls) return fail(KV_ERR_ARG, "pool, total_ms and n_calls are required");
  double sum = 0.0;
  for (size_t i = 0; i < pool->timing_used; ++i) {
    hipError_t e = hipEventSynchronize(pool->timing[i].second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pool->timing[i].first, pool->timing[i].second);
    if (e != hipSuccess) return hip_fail(e, "timing events");
    sum += ms;
  }
  *total_ms = sum;
  *n_calls = (int32_t)pool->timing_used;
  return ok();
}

kv_status kv_pool_destroy(kv_pool_t* pool) {
  if (!pool) return fail(KV_ERR_ARG, "pool is NULL");
  free_timing(pool);
  discard_pending(pool);
  for (auto& ps : pool->pending)
    if (ps.done) (void)hipEventDestroy(ps.done);
  if (pool->pinned) (void)hipHostFree(pool->pinned);
  if (pool->slots) (void)hipHostFree(pool->slots);
  if (pool->div_staged) (void)hipEventDestroy(pool->div_staged);
  if (pool->wait_ev) (void)hipEventDestroy(pool->wait_ev);
  if (pool->div_pinned) (void)hipHostFree(pool->div_pinned);
  delete pool;
  return ok();
}

kv_status kv_reset(kv_pool_t* pool) {
  if (!pool) return fail(KV_ERR_ARG, "pool is NULL");
  discard_pending(pool);
  for (auto& l : pool->layers) l.reset();
  for (auto& r : pool->rank_slots) r.valid = false;
  return ok();
}

kv_status kv_sync(kv_pool_t* pool, int32_t layer) {
  if (!pool) return fail(KV_ERR_ARG, "pool is NULL");
  if (layer == -1) {
    kv_status first_err = KV_OK;
    std::string msg;
    for (int32_t l = 0; l < pool->cfg.num_layers; ++l) {
      kv_status s = settle(pool, l);
      if (s != KV_OK && first_err == KV_OK) {
        first_err = s;
        msg = g_err;
      }
    }
    if (first_err != KV_OK) {
      g_err = msg;
      return first_err;
    }
    return ok();
  }
  kv_status s = check_layer(pool, layer);
  return s != KV_OK ? s : ok();
}

kv_status kv_append_frame(kv_pool_t* pool, int32_t layer, int64_t frame_idx, const void* k_dev, const void* v_dev,
                          int32_t n_tokens, uint32_t flags, void* stream) {
  kv_status s = check_layer(pool, layer);
  if (s != KV_OK) return s;
  if (n_tokens != pool->cfg.page_tokens)
    return fail(KV_ERR_SHAPE, "n_tokens %d != page_tokens %d", n_tokens, pool->cfg.page_tokens);
  if (frame_idx < 0) return fail(KV_ERR_ARG, "negative frame index");
  if (frame_idx > (int64_t)(INT32_MAX / pool->cfg.page_tokens) - 1)
    return fail(KV_ERR_ARG, "frame index %lld too large for 32-bit token ids", (long long)frame_idx);
  if (flags & ~KV_TRANSIENT) return fail(KV_ERR_ARG, "unknown flags 0x%x", flags);
  auto& L = pool->layers[(size_t)layer];
  int32_t page = 0;
  int rc = L.plan_append(frame_idx, (flags & KV_TRANSIENT) != 0, &page);
  if (rc == 1)
    return fail(KV_ERR_STATE, "layer %d: frame %lld after frame %lld%s", layer, (long long)frame_idx,
                (long long)L.last_frame, L.transient_pending ? " (a transient frame is still pending)" : "");
  if (rc == 2) return fail(KV_ERR_NO_PAGES, "layer %d: all %d page ids in use", layer, pool->cfg.pages_per_layer);
  if (!pool->meta_only) {
    if (!k_dev || !v_dev) return fail(KV_ERR_ARG, "k or v is NULL");
    char* dst = pool->pool + phys_page(pool, layer, page) * pool->lay.geom.page_bytes;
    hipError_t e = kvs::launch_append(pool->lay.geom, dst, k_dev, v_dev, n_tokens,
                                      frame_idx * pool->cfg.page_tokens, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "page write launch");
  }
  L.commit_append(frame_idx, page);
  return ok();
}

kv_status kv_append_frame_layers(kv_pool_t* pool, int32_t first_layer, int32_t n_layers, int64_t frame_idx,
                                 const void* k_dev, const void* v_dev, int32_t n_tokens, uint32_t flags,
                                 void* stream) {
  kv_status s = check_layers(pool, first_layer, n_layers);  // completes deferred steps of these layers
  if (s != KV_OK) return s;
  if (n_tokens != pool->cfg.page_tokens)
    return fail(KV_ERR_SHAPE, "n_tokens %d != page_tokens %d", n_tokens, pool->cfg.page_tokens);
  if (frame_idx < 0) return fail(KV_ERR_ARG, "negative frame index");
  if (frame_idx > (int64_t)(INT32_MAX / pool->cfg.page_tokens) - 1)
    return fail(KV_ERR_ARG, "frame index %lld too large for 32-bit token ids", (long long)frame_idx);
  if (flags & ~KV_TRANSIENT) return fail(KV_ERR_ARG, "unknown flags 0x%x", flags);
  std::vector<int32_t> pages((size_t)n_layers);
  for (int32_t i = 0; i < n_layers; ++i) {  // check every layer before changing any
    auto& L = pool->layers[(size_t)(first_layer + i)];
    int rc = L.plan_append(frame_idx, (flags & KV_TRANSIENT) != 0, &pages[(size_t)i]);
    if (rc == 1)
      return fail(KV_ERR_STATE, "layer %d: frame %lld after frame %lld%s", first_layer + i, (long long)frame_idx,
                  (long long)L.last_frame, L.transient_pending ? " (a transient frame is still pending)" : "");
    if (rc == 2)
      return fail(KV_ERR_NO_PAGES, "layer %d: all %d page ids in use", first_layer + i, pool->cfg.pages_per_layer);
  }
  if (!pool->meta_only) {
    if (!k_dev || !v_dev) return fail(KV_ERR_ARG, "k or v is NULL");
    const int64_t frame_bytes = (int64_t)n_tokens * pool->cfg.num_heads * kvs::kHeadDim * pool->lay.geom.esize;
    for (int32_t c0 = 0; c0 < n_layers; c0 += kvs::kAppendLayersChunk) {
      const int32_t nc = std::min<int32_t>(kvs::kAppendLayersChunk, n_layers - c0);
      kvs::AppendLayers al;
      for (int32_t i = 0; i < nc; ++i)
        al.page_offset[i] = phys_page(pool, first_layer + c0 + i, pages[(size_t)(c0 + i)]) * pool->lay.geom.page_bytes;
      hipError_t e = kvs::launch_append_layers(pool->lay.geom, pool->pool, al, nc,
                                               static_cast<const char*>(k_dev) + c0 * frame_bytes,
                                               static_cast<const char*>(v_dev) + c0 * frame_bytes, n_tokens,
                                               frame_idx * pool->cfg.page_tokens, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return hip_fail(e, "multi-layer page write launch");
    }
  }
  for (int32_t i = 0; i < n_layers; ++i) pool->layers[(size_t)(first_layer + i)].commit_append(frame_idx, pages[(size_t)i]);
  return ok();
}

namespace {

// Copies of the special rows of evicted frames into the special pages.  A
// copy whose destination is the source of an earlier copy in the same launch
// (a victim's freed id reused as a special page) starts a new launch, which
// the stream orders after it.
kv_status launch_special_copies(kv_pool_t* pool, int32_t layer, const std::vector<kvs::MergeMove>& mv,
                                hipStream_t st) {
  const int64_t pb = pool->lay.geom.page_bytes;
  kvs::MergeChunk c;
  c.n = 0;
  std::set<int32_t> sources;
  hipError_t e = hipSuccess;
  auto flush = [&]() {
    if (c.n > 0 && e == hipSuccess) e = kvs::launch_merge(pool->lay.geom, pool->pool, c, st);
    c.n = 0;
    sources.clear();
  };
  for (const auto& m : mv) {
    if (c.n == kvs::kMergeChunk || sources.count(m.dst)) flush();
    c.item[c.n].src_offset = phys_page(pool, layer, m.src) * pb;
    c.item[c.n].dst_offset = phys_page(pool, layer, m.dst) * pb;
    c.item[c.n].dst_off = m.dst_off;
    c.item[c.n].count = m.count;
    ++c.n;
    sources.insert(m.src);
  }
  flush();
  return e == hipSuccess ? KV_OK : hip_fail(e, "special-token copy launch");
}

}  // namespace

kv_status kv_evict(kv_pool_t* pool, int32_t layer, int32_t* n_evicted, void* stream) {
  kv_status s = check_layer(pool, layer);
  if (s != KV_OK) return s;
  auto& L = pool->layers[(size_t)layer];
  // the special-token copies are launched after the policy changed: keep the
  // old state to restore if a launch fails (only then is there device work)
  std::unique_ptr<kvs::LayerPolicy> saved;
  if (pool->cfg.special_tokens > 0 && !pool->meta_only) saved.reset(new kvs::LayerPolicy(L));
  std::vector<kvs::MergeMove> mv;
  const int32_t n = L.evict(&mv);
  if (n < 0)
    return fail(KV_ERR_NO_PAGES, "layer %d: no free page id for the special tokens of an evicted frame", layer);
  if (!pool->meta_only && !mv.empty()) {
    s = launch_special_copies(pool, layer, mv, static_cast<hipStream_t>(stream));
    if (s != KV_OK) {
      L = *saved;
      return s;
    }
  }
  if (n_evicted) *n_evicted = n;
  return ok();
}

kv_status kv_set_attend_tiling(kv_pool_t* pool, int32_t tiling) {
  if (!pool) return fail(KV_ERR_ARG, "pool is NULL");
  if (tiling != KV_TILING_AUTO && tiling != KV_TILING_PAGE && tiling != KV_TILING_PACKED)
    return fail(KV_ERR_ARG, "tiling %d is none of KV_TILING_AUTO, KV_TILING_PAGE, KV_TILING_PACKED", tiling);
  pool->tiling = tiling;
  return ok();
}

kv_status kv_set_attend_splits(kv_pool_t* pool, int32_t splits) {
  if (!pool) return fail(KV_ERR_ARG, "pool is NULL");
  if (splits < 0 || splits > pool->cfg.max_splits) return fail(KV_ERR_ARG, "splits %d out of 0..max_splits", splits);
  pool->splits_override = splits;
  return ok();
}

namespace {

kv_status check_attend_args(const kv_pool_t* pool, const void* q_dev, int32_t n_q, float sm_scale,
                            const void* out_dev) {
  if (n_q < 1 || n_q > pool->cfg.max_queries)
    return fail(KV_ERR_SHAPE, "n_q %d out of 1..max_queries (%d)", n_q, pool->cfg.max_queries);
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return fail(KV_ERR_ARG, "sm_scale must be finite and > 0");
  if (pool->meta_only) return fail(KV_ERR_STATE, "metadata-only pool has no device memory");
  if (!q_dev || !out_dev) return fail(KV_ERR_ARG, "q or out is NULL");
  return KV_OK;
}

// A page write that rides in the table-upload launch of the attention.
struct PageWrite {
  const void* k;
  const void* v;
  char* page;
  int64_t first_id;
};

// Uploads the table of L (the layer's policy, possibly a not yet committed
// copy) and launches the attention over it; with `write`, the frame's page
// write and the table upload are one launch, ordered before the attention.
// Changes no host state.
kv_status attend_launch(kv_pool_t* pool, int32_t layer, const kvs::LayerPolicy& L, const void* q_dev, int32_t n_q,
                        float sm_scale, void* out_dev, float* lse_dev, hipStream_t st, const PageWrite* write,
                        bool static_scratch = false) {
  auto& ent = pool->scratch;
  ent.clear();
  const int32_t H = pool->cfg.num_heads;
  const bool per_head = !L.same_lengths();
  // The shared table: one entry per page with tokens (the longest head's
  // length).  Once heads hold different counts, every page stays in it,
  // flagged (tile_start = 1) where its per-head lengths live in the device
  // array the prune wrote, and one table per head is built from it on the
  // device, each ending with an entry that carries the head's tile count.
  int32_t tiles = 0, toks = 0;
  auto add = [&](int32_t page, int32_t len, int32_t flag) {
    kvs::DevEntry d;
    d.phys = (int32_t)phys_page(pool, layer, page);
    d.len = len;
    d.tile_start = per_head ? flag : tiles;
    d.tok_start = toks;
    tiles += (len + kvs::kTile - 1) / kvs::kTile;
    toks += len;
    ent.push_back(d);
  };
  for (const auto& e : L.table)
    if (per_head || e.len > 0) add(e.page, e.len, e.hlen.empty() ? 0 : 1);
  if (L.transient_pending) add(-1, pool->cfg.page_tokens, 0);
  const int32_t n_entries = (int32_t)ent.size();
  // Tiles per page, or packed over each head's tokens across page ends.
  // Automatic: packed for per-head tables whose per-page tiles leave more than
  // 3% of the slots empty.  There the heads hold equal token counts spread
  // over their pages differently, so per-page tiles give the most fragmented
  // head the most tiles, and its workgroups set the kernel's time; packed
  // tiles even the heads out.  A shared table gives every head the same tiles,
  // and packing only trades the pages' partial tiles for tiles that span page
  // ends (about even at a budget cache's 340-token pages, a loss at full
  // 1004-token pages).
  auto packed_tiles = [](int64_t tokens) { return (int32_t)((tokens + kvs::kTile - 1) / kvs::kTile); };
  int64_t page_tiles_all = tiles, packed_tiles_all = packed_tiles(toks);
  int32_t min_page_tiles = tiles, min_packed_tiles = packed_tiles(toks);
  if (per_head) {
    page_tiles_all = packed_tiles_all = 0;
    min_page_tiles = min_packed_tiles = INT32_MAX;
    for (int32_t h = 0; h < H; ++h) {
      int32_t t_h = 0, tok_h = 0;
      for (const auto& e : L.table) {
        const int32_t n = kvs::head_len(e, h);
        t_h += (n + kvs::kTile - 1) / kvs::kTile;
        tok_h += n;
      }
      if (L.transient_pending) {
        t_h += (pool->cfg.page_tokens + kvs::kTile - 1) / kvs::kTile;
        tok_h += pool->cfg.page_tokens;
      }
      page_tiles_all += t_h;
      packed_tiles_all += packed_tiles(tok_h);
      min_page_tiles = std::min(min_page_tiles, t_h);
      min_packed_tiles = std::min(min_packed_tiles, packed_tiles(tok_h));
    }
  }
  const bool packed = pool->tiling == KV_TILING_AUTO ? per_head && packed_tiles_all * 103 < page_tiles_all * 100
                                                      : pool->tiling == KV_TILING_PACKED;
  const int32_t min_tiles = packed ? min_packed_tiles : min_page_tiles;
  if (n_entries == 0 || min_tiles == 0) return fail(KV_ERR_STATE, "layer %d holds no token to attend to", layer);

  const bool bf16 = pool->cfg.dtype == KV_BF16;
  int32_t splits = 1;
  if (bf16) {
    const int64_t qtiles = (n_q + kvs::kAttendRows - 1) / kvs::kAttendRows;
    const int64_t base = qtiles * pool->cfg.num_heads;
    if (pool->splits_override > 0) {
      splits = pool->splits_override;
    } else {
      // one full round of resident workgroups (256 CUs x 2): split counts that
      // leave a partial round run measurably slower, and fewer splits write
      // fewer partials for the combine
      const int64_t target = 512;
      splits = (int32_t)std::max<int64_t>(1, (target + base / 2) / base);
    }
    splits = std::min<int32_t>(splits, pool->cfg.max_splits);
    splits = std::min<int32_t>(splits, min_tiles);
    splits = (int32_t)std::min<int64_t>(splits, std::max<int64_t>(1, pool->lay.part_rows / n_q));
    splits = std::max(splits, 1);
  }
  // split-KV partials: the pool's workspace, or this GPU's static scratch
  float* part_o = reinterpret_cast<float*>(pool->ws + pool->lay.part_o);
  float* part_ml = reinterpret_cast<float*>(pool->ws + pool->lay.part_ml);
  if (static_scratch && splits > 1) {
    const size_t o_bytes = align_up((size_t)splits * (size_t)n_q * (size_t)H * kvs::kHeadDim * 4);
    const size_t need = o_bytes + (size_t)splits * (size_t)n_q * (size_t)H * 2 * 4;
    if (need > kvs::kAttendScratchBytes)
      return fail(KV_ERR_SHAPE, "split-KV partials of %zu bytes (%d splits x %d queries x %d heads) exceed the "
                  "%zu-byte static scratch", need, splits, n_q, H, kvs::kAttendScratchBytes);
    char* base = nullptr;
    hipError_t se = kvs::attend_scratch_address(&base);
    if (se != hipSuccess) return hip_fail(se, "static scratch address");
    part_o = reinterpret_cast<float*>(base);
    part_ml = reinterpret_cast<float*>(base + o_bytes);
  }
  kvs::DevEntry* dt = dev_table(pool, layer);
  hipError_t e = hipSuccess;
  // per-head tables are built on the device from the shared one, uploaded after them
  kvs::DevEntry* up = per_head ? dt + (int64_t)H * (pool->lay.layer_pages + 1) : dt;
  // a short shared table rides in the attention launch's arguments: no upload launch
  const bool inline_table = bf16 && !per_head && !write && n_entries <= kvs::kUploadChunk;
  kvs::TableChunk chunk;
  if (inline_table) {
    chunk.first = 0;
    chunk.count = n_entries;
    std::copy(ent.begin(), ent.begin() + n_entries, chunk.e);
  } else if (write) {
    e = kvs::launch_append_table(pool->lay.geom, write->page, write->k, write->v, pool->cfg.page_tokens,
                                 write->first_id, up, ent.data(), n_entries, st);
  } else {
    e = kvs::launch_table_upload(up, ent.data(), n_entries, st);
  }
  if (e == hipSuccess && per_head) e = kvs::launch_head_tables(dt, up, n_entries, hlens_dev(pool), H, st);
  if (e != hipSuccess) return hip_fail(e, write ? "page write and table upload launch" : "table upload launch");

  kvs::AttendParams ap{};
  ap.q = q_dev;
  ap.out = out_dev;
  ap.lse = lse_dev;
  ap.part_o = part_o;
  ap.part_ml = part_ml;
  ap.pool = pool->pool;
  ap.table = dt;
  ap.n_entries = n_entries;
  ap.total_tiles = tiles;
  ap.total_tokens = toks;
  ap.packed = packed ? 1 : 0;
  ap.inline_table = inline_table ? 1 : 0;
  ap.head_stride = per_head ? n_entries + 1 : 0;
  ap.splits = splits;
  ap.n_q = n_q;
  ap.scale_log2 = sm_scale * 1.4426950408889634f;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (pool->timing_used < pool->timing.size()) {
    ev0 = pool->timing[pool->timing_used].first;
    ev1 = pool->timing[pool->timing_used].second;
    ++pool->timing_used;
  }
  e = kvs::launch_attend(pool->lay.geom, ap, bf16, st, ev0, ev1, inline_table ? &chunk : nullptr);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return KV_OK;
}

}  // namespace

kv_status stream_attend(kv_pool_t* pool, int32_t layer, const void* q_dev, int32_t n_q, float sm_scale,
                        void* out_dev, float* lse_dev, void* stream) {
  kv_status s = check_layer(pool, layer);
  if (s != KV_OK) return s;
  s = check_attend_args(pool, q_dev, n_q, sm_scale, out_dev);
  if (s != KV_OK) return s;
  auto& L = pool->layers[(size_t)layer];
  s = attend_launch(pool, layer, L, q_dev, n_q, sm_scale, out_dev, lse_dev, static_cast<hipStream_t>(stream),
                    nullptr);
  if (s != KV_OK) return s;
  L.transient_pending = false;
  return ok();
}

kv_status stream_attend_scratch(kv_pool_t* pool, int32_t layer, const void* q_dev, int32_t n_q, float sm_scale,
                                void* out_dev, float* lse_dev, void* stream) {
  kv_status s = check_layer(pool, layer);
  if (s != KV_OK) return s;
  s = check_attend_args(pool, q_dev, n_q, sm_scale, out_dev);
  if (s != KV_OK) return s;
  auto& L = pool->layers[(size_t)layer];
  s = attend_launch(pool, layer, L, q_dev, n_q, sm_scale, out_dev, lse_dev, static_cast<hipStream_t>(stream),
                    nullptr, true);
  if (s != KV_OK) return s;
  L.transient_pending = false;
  return ok();
}

kv_status kv_append_attend(kv_pool_t* pool, int32_t layer, int64_t frame_idx, const void* k_dev, const void* v_dev,
                           int32_t n_tokens, uint32_t flags, const void* q_dev, int32_t n_q, float sm_scale,
                           void* out_dev, float* lse_dev, int32_t* n_evicted, void* stream) {
  kv_status s = check_layer(pool, layer);
  if (s != KV_OK) return s;
  if (n_tokens != pool->cfg.page_tokens)
    return fail(KV_ERR_SHAPE, "n_tokens %d != page_tokens %d", n_tokens, pool->cfg.page_tokens);
  if (frame_idx < 0) return fail(KV_ERR_ARG, "negative frame index");
  if (frame_idx > (int64_t)(INT32_MAX / pool->cfg.page_tokens) - 1)
    return fail(KV_ERR_ARG, "frame index %lld too large for 32-bit token ids", (long long)frame_idx);
  if (flags & ~KV_TRANSIENT) return fail(KV_ERR_ARG, "unknown flags 0x%x", flags);
  s = check_attend_args(pool, q_dev, n_q, sm_scale, out_dev);
  if (s != KV_OK) return s;
  if (!k_dev || !v_dev) return fail(KV_ERR_ARG, "k or v is NULL");
  auto& L = pool->layers[(size_t)layer];
  int32_t page = 0;
  int rc = L.plan_append(frame_idx, (flags & KV_TRANSIENT) != 0, &page);
  if (rc == 1)
    return fail(KV_ERR_STATE, "layer %d: frame %lld after frame %lld%s", layer, (long long)frame_idx,
                (long long)L.last_frame, L.transient_pending ? " (a transient frame is still pending)" : "");
  if (rc == 2) return fail(KV_ERR_NO_PAGES, "layer %d: all %d page ids in use", layer, pool->cfg.pages_per_layer);

  // the append and the eviction act on a copy that replaces the layer's
  // policy only once every launch is enqueued
  kvs::LayerPolicy next = L;
  next.commit_append(frame_idx, page);
  std::vector<kvs::MergeMove> mv;
  const int32_t n_ev = next.evict(&mv);
  if (n_ev < 0)
    return fail(KV_ERR_NO_PAGES, "layer %d: no free page id for the special tokens of an evicted frame", layer);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!mv.empty()) {
    s = launch_special_copies(pool, layer, mv, st);
    if (s != KV_OK) return s;
  }
  const PageWrite w{k_dev, v_dev, pool->pool + phys_page(pool, layer, page) * pool->lay.geom.page_bytes,
                    frame_idx * pool->cfg.page_tokens};
  s = attend_launch(pool, layer, next, q_dev, n_q, sm_scale, out_dev, lse_dev, st, &w);
  if (s != KV_OK) return s;
  next.transient_pending = false;
  L = std::move(next);
  if (n_evicted) *n_evicted = n_ev;
  return ok();
}

kv_status score_and_compact(kv_pool_t* pool, int32_t layer, const float* score_table_dev, int64_t score_rows,
                            const kv_clces_params* params, int32_t* keep_ids_out_dev, int32_t* ranks_out_dev,
                            int64_t* n_kept, void* stream) {
  kv_status s = check_layer(pool, layer);
  if (s != KV_OK) return s;
  if (!params) return fail(KV_ERR_ARG, "params is NULL");
  if (params->window < 1 || params->window > pool->cfg.max_window)
    return fail(KV_ERR_ARG, "window %d out of 1..max_window (%d)", params->window, pool->cfg.max_window);
  if (!std::isfinite(params->lambda) || params->lambda < 0) return fail(KV_ERR_ARG, "lambda must be finite and >= 0");
  if (params->keep_count < 0) return fail(KV_ERR_ARG, "keep_count must be >= 0");
  if (params->flags & ~(KV_CLCES_DEFER | KV_CLCES_REUSE_RANKS | KV_CLCES_RANK_RADIX))
    return fail(KV_ERR_ARG, "unknown CLCES flags 0x%x", params->flags);
  auto& L = pool->layers[(size_t)layer];
  if (!L.same_tokens()) return fail(KV_ERR_STATE, "layer %d: heads hold different tokens (diversity-pruned)", layer);
  if (pool->cfg.special_tokens > 0)
    return fail(KV_ERR_STATE, "compaction would move the special tokens out of a frame's first slots "
                              "(special_tokens > 0)");
  const size_t first = L.first_candidate();
  int64_t N = 0;
  for (size_t i = first; i < L.table.size(); ++i) N += L.table[i].len;
  if (N <= params->keep_count) {
    if (n_kept) *n_kept = N;
    return ok();
  }
  if (pool->meta_only) return fail(KV_ERR_STATE, "metadata-only pool has no device memory");
  if (!score_table_dev) return fail(KV_ERR_ARG, "score table is NULL");
  if (score_rows < 1) return fail(KV_ERR_ARG, "score_rows must be >= 1");

  auto& ent = pool->scratch;
  ent.clear();
  int32_t toks = 0;
  for (size_t i = first; i < L.table.size(); ++i) {
    kvs::DevEntry d;
    d.phys = (int32_t)phys_page(pool, layer, L.table[i].page);
    d.len = L.table[i].len;
    d.tile_start = 0;
    d.tok_start = toks;
    toks += d.len;
    ent.push_back(d);
  }
  const int32_t n_win = std::min<int32_t>(params->window, layer + 1);
  kvs::ClcesArgs a{};
  a.ws = pool->ws + pool->lay.clces;
  a.sizes = pool->lay.cl;
  a.pool = pool->pool;
  a.geom = pool->lay.geom;
  a.entries_host = ent.data();
  a.n_entries = (int32_t)ent.size();
  a.n_tokens = (int32_t)N;
  a.score_table = score_table_dev;
  a.score_rows = score_rows;
  a.score_cols = pool->cfg.num_layers;
  a.first_layer = layer - n_win + 1;
  a.n_window = n_win;
  a.lambda = params->lambda;
  a.rank_radix = (params->flags & KV_CLCES_RANK_RADIX) != 0;
  a.keep = params->keep_count;
  a.keep_ids_out = keep_ids_out_dev;
  a.s_hat_out = params->s_hat_out;
  // Rank history ([SCV] 2.1.4): with KV_CLCES_REUSE_RANKS, a window layer
  // whose ranks an earlier synchronous step computed over the same candidate
  // sequence (a layer never compacted, merged or pruned holds whole frames, so
  // its candidate frames name the sequence) and the same score table is not
  // ranked again.  Every other window layer is ranked into the least recently
  // used slot not taken by this step.
  const bool pristine = L.compactions == 0 && L.merges == 0 && L.prunes == 0;
  const bool reuse = (params->flags & KV_CLCES_REUSE_RANKS) != 0 && pristine;
  std::vector<int64_t> frames;
  if (reuse)
    for (size_t i = first; i < L.table.size(); ++i) frames.push_back(L.table[i].frame);
  auto& slots = pool->rank_slots;
  std::vector<char> taken(slots.size(), 0);
  std::vector<int32_t> slot_of((size_t)n_win, -1);
  const uint64_t now = ++pool->rank_clock;
  for (int32_t w = 0; w < n_win && reuse; ++w)
    for (size_t k = 0; k < slots.size(); ++k) {
      const auto& r = slots[k];
      if (r.valid && r.column == a.first_layer + w && r.table == score_table_dev && r.rows == score_rows &&
          r.frames == frames) {
        slot_of[(size_t)w] = (int32_t)k;
        taken[k] = 1;
        break;
      }
    }
  a.n_rank = 0;
  for (int32_t w = 0; w < n_win; ++w) {
    if (slot_of[(size_t)w] < 0) {
      size_t best = slots.size();
      for (size_t k = 0; k < slots.size(); ++k)
        if (!taken[k] && (best == slots.size() || !slots[k].valid ||
                          (slots[best].valid && slots[k].used < slots[best].used)))
          best = k;
      slot_of[(size_t)w] = (int32_t)best;
      taken[best] = 1;
      slots[best].valid = false;  // overwritten by this step
      a.rank_new[w] = 1;
      ++a.n_rank;
    }
    slots[(size_t)slot_of[(size_t)w]].used = now;
    a.rank_dst[w] = reinterpret_cast<int32_t*>(pool->ws + pool->lay.rank_cache) +
                    (int64_t)slot_of[(size_t)w] * pool->cfg.pages_per_layer * pool->cfg.page_tokens;
  }
  auto copy_ranks = [&](hipStream_t st) -> hipError_t {
    for (int32_t w = 0; w < n_win && ranks_out_dev; ++w) {
      hipError_t ce = hipMemcpyAsync(ranks_out_dev + (int64_t)w * N, a.rank_dst[w], sizeof(int32_t) * (size_t)N,
                                     hipMemcpyDeviceToDevice, st);
      if (ce != hipSuccess) return ce;
    }
    return hipSuccess;
  };
  auto record_ranks = [&]() {
    if (!reuse) return;
    for (int32_t w = 0; w < n_win; ++w)
      if (a.rank_new[w]) {
        auto& r = slots[(size_t)slot_of[(size_t)w]];
        r.valid = true;
        r.column = a.first_layer + w;
        r.table = score_table_dev;
        r.rows = score_rows;
        r.frames = frames;
      }
  };
  if (params->flags & KV_CLCES_DEFER) {
    // enqueue the step and its read-back; the next call on this layer applies it
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto& ps = pool->pending[(size_t)layer];
    hipError_t e = hipSuccess;
    if (!pool->pinned) e = clces_pinned(pool);
    if (e == hipSuccess && !ps.done) e = hipEventCreateWithFlags(&ps.done, hipEventDisableTiming);
    if (e == hipSuccess) e = kvs::enqueue_clces(a, st);
    if (e == hipSuccess) e = copy_ranks(st);
    if (e == hipSuccess)
      e = hipMemcpyAsync(pool->pinned + (size_t)layer * ((size_t)pool->cfg.pages_per_layer + 1), kvs::clces_result(a),
                         sizeof(int32_t) * ((size_t)a.n_entries + 1), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipEventRecord(ps.done, st);
    if (e != hipSuccess) return hip_fail(e, "deferred CLCES step");
    ps.active = true;
    ps.n_entries = a.n_entries;
    ps.keep = params->keep_count;
    if (n_kept) *n_kept = params->keep_count;
    return ok();
  }
  std::vector<int32_t> new_lens((size_t)a.n_entries);
  int32_t err_flag = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the index step writes each page's new length (or the error flag) into
  // the pool's page words as soon as it is known; the host waits for those
  // words only, while the rows move
  hipError_t e = pool->slots ? hipSuccess : clces_slots(pool);
  if (++pool->slot_seq == 0) pool->slot_seq = 1;
  a.host_slots = pool->slots_dev;
  a.slot_seq = pool->slot_seq;
  if (e == hipSuccess) e = kvs::enqueue_clces(a, st);
  if (e == hipSuccess) e = copy_ranks(st);
  bool complete = false;
  if (e == hipSuccess) e = wait_slots(pool, st, a.n_entries, &complete);
  if (e != hipSuccess) return hip_fail(e, "CLCES step");
  if (!complete) return fail(KV_ERR_HIP, "layer %d: the CLCES step did not report every page's length", layer);
  for (int32_t i = 0; i < a.n_entries; ++i) {
    const uint32_t v = (uint32_t)(pool->slots[i] & 0xffffffffu);
    if (v & kvs::kSlotError)
      err_flag |= (int32_t)(v & ~kvs::kSlotError);
    else
      new_lens[(size_t)i] = (int32_t)v;
  }
  if (err_flag & kvs::kClcesErrNan) return fail(KV_ERR_NAN, "layer %d: a raw score is NaN or negative", layer);
  if (err_flag & kvs::kClcesErrRow) return fail(KV_ERR_ARG, "layer %d: a token id is >= score_rows", layer);
  if (err_flag) return fail(KV_ERR_HIP, "layer %d: CLCES consistency check failed (flag %d)", layer, err_flag);
  int64_t kept = 0;
  for (int32_t v : new_lens) kept += v;
  if (kept != params->keep_count)
    return fail(KV_ERR_HIP, "layer %d: kept %lld tokens, expected %lld", layer, (long long)kept,
                (long long)params->keep_count);
  record_ranks();
  L.apply_compaction(new_lens, kept);
  if (n_kept) *n_kept = kept;
  return ok();
}

namespace {

// Page merges of layers first .. first+n-1: each layer's plan (whole pages
// where every head holds the same rows, per head otherwise), the moves of all
// layers packed into shared launches (moves carry absolute page offsets; a
// plan never moves a page it writes), then every layer's table updated.
kv_status merge_layers(kv_pool_t* pool, int32_t first, int32_t n, int32_t* n_merged, hipStream_t st) {
  if (pool->cfg.sliding_window > 0)
    return fail(KV_ERR_STATE, "page merge needs one frame per page no more (sliding_window must be 0)");
  const int32_t H = pool->cfg.num_heads;
  std::vector<std::vector<kvs::MergeMove>> whole((size_t)n);
  std::vector<std::vector<kvs::HeadMergeMove>> heads((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    const auto& L = pool->layers[(size_t)(first + i)];
    if (L.same_tokens()) {
      whole[(size_t)i] = L.plan_merges();
    } else {
      if (2 * H > kvs::kHeadMergeInts)
        return fail(KV_ERR_ARG, "per-head page merge supports at most %d heads", kvs::kHeadMergeInts / 2);
      heads[(size_t)i] = L.plan_head_merges(H);
    }
  }
  if (!pool->meta_only) {
    const int64_t pb = pool->lay.geom.page_bytes;
    hipError_t e = hipSuccess;
    kvs::MergeChunk c;
    c.n = 0;
    for (int32_t i = 0; i < n && e == hipSuccess; ++i)
      for (const auto& m : whole[(size_t)i]) {
        c.item[c.n].src_offset = phys_page(pool, first + i, m.src) * pb;
        c.item[c.n].dst_offset = phys_page(pool, first + i, m.dst) * pb;
        c.item[c.n].dst_off = m.dst_off;
        c.item[c.n].count = m.count;
        if (++c.n == kvs::kMergeChunk) {
          e = kvs::launch_merge(pool->lay.geom, pool->pool, c, st);
          c.n = 0;
          if (e != hipSuccess) break;
        }
      }
    if (e == hipSuccess && c.n > 0) e = kvs::launch_merge(pool->lay.geom, pool->pool, c, st);
    // per-head moves; the last move into each destination writes its per-head lengths
    const int per_chunk = (int)std::min<int64_t>(kvs::kHeadMergeItems, kvs::kHeadMergeInts / (2 * (int64_t)H));
    kvs::HeadMergeChunk hc;
    hc.n = 0;
    std::vector<size_t> last_into((size_t)pool->cfg.pages_per_layer);
    for (int32_t i = 0; i < n && e == hipSuccess; ++i) {
      const auto& mv = heads[(size_t)i];
      for (size_t j = 0; j < mv.size(); ++j) last_into[(size_t)mv[j].dst] = j;
      for (size_t j = 0; j < mv.size(); ++j) {
        const auto& m = mv[j];
        const int k = hc.n;
        hc.src_offset[k] = phys_page(pool, first + i, m.src) * pb;
        hc.dst_offset[k] = phys_page(pool, first + i, m.dst) * pb;
        hc.dst_phys[k] = (int32_t)phys_page(pool, first + i, m.dst);
        hc.last[k] = last_into[(size_t)m.dst] == j ? 1 : 0;
        for (int32_t h = 0; h < H; ++h) {
          hc.hv[2 * (k * H + h)] = m.dst_off[(size_t)h];
          hc.hv[2 * (k * H + h) + 1] = m.count[(size_t)h];
        }
        if (++hc.n == per_chunk) {
          e = kvs::launch_head_merge(pool->lay.geom, pool->pool, hlens_dev(pool), hc, st);
          hc.n = 0;
          if (e != hipSuccess) break;
        }
      }
    }
    if (e == hipSuccess && hc.n > 0) e = kvs::launch_head_merge(pool->lay.geom, pool->pool, hlens_dev(pool), hc, st);
    if (e != hipSuccess) return hip_fail(e, "page merge launch");
  }
  for (int32_t i = 0; i < n; ++i) {
    auto& L = pool->layers[(size_t)(first + i)];
    const size_t moved = whole[(size_t)i].size() + heads[(size_t)i].size();
    if (!whole[(size_t)i].empty()) L.commit_merges(whole[(size_t)i]);
    if (!heads[(size_t)i].empty()) L.commit_head_merges(heads[(size_t)i], H);
    if (n_merged) n_merged[i] = (int32_t)moved;
  }
  return ok();
}

}  // namespace

kv_status kv_merge_pages(kv_pool_t* pool, int32_t layer, int32_t* n_merged, void* stream) {
  kv_status s = check_layer(pool, layer);
  if (s != KV_OK) return s;
  return merge_layers(pool, layer, 1, n_merged, static_cast<hipStream_t>(stream));
}

kv_status kv_merge_pages_layers(kv_pool_t* pool, int32_t first_layer, int32_t n_layers, int32_t* n_merged,
                                void* stream) {
  kv_status s = check_layers(pool, first_layer, n_layers);
  if (s != KV_OK) return s;
  return merge_layers(pool, first_layer, n_layers, n_merged, static_cast<hipStream_t>(stream));
}

kv_status kv_diversity_score(kv_pool_t* pool, int32_t layer, double* scores_dev, int64_t score_stride,
                             double* mean_diversity, void* stream) {
  kv_status s = check_layer(pool, layer);
  if (s != KV_OK) return s;
  if (!mean_diversity) return fail(KV_ERR_ARG, "mean_diversity is NULL");
  return diversity_score_range(pool, layer, 1, scores_dev, score_stride, mean_diversity,
                               static_cast<hipStream_t>(stream));
}

kv_status kv_diversity_score_layers(kv_pool_t* pool, int32_t first_layer, int32_t n_layers, double* mean_diversity,
                                    void* stream) {
  kv_status s = check_layers(pool, first_layer, n_layers);
  if (s != KV_OK) return s;
  if (!mean_diversity) return fail(KV_ERR_ARG, "mean_diversity is NULL");
  return diversity_score_range(pool, first_layer, n_layers, nullptr, 0, mean_diversity,
                               static_cast<hipStream_t>(stream));
}

kv_status kv_diversity_prune(kv_pool_t* pool, int32_t layer, int64_t keep_per_head, double* scores_dev,
                             int64_t score_stride, int64_t* kept_per_head, void* stream) {
  kv_status s = check_layer(pool, layer);
  if (s != KV_OK) return s;
  return diversity_prune_range(pool, layer, 1, &keep_per_head, scores_dev, score_stride, kept_per_head,
                               static_cast<hipStream_t>(stream));
}

kv_status kv_diversity_prune_layers(kv_pool_t* pool, int32_t first_layer, int32_t n_layers,
                                    const int64_t* keep_per_head, int64_t* kept_per_head, void* stream) {
  kv_status s = check_layers(pool, first_layer, n_layers);
  if (s != KV_OK) return s;
  if (!keep_per_head) return fail(KV_ERR_ARG, "keep_per_head is NULL");
  return diversity_prune_range(pool, first_layer, n_layers, keep_per_head, nullptr, 0, kept_per_head,
                               static_cast<hipStream_t>(stream));
}

kv_status kv_layer_budgets(const double* mean_diversity, int32_t n_layers, double tau, int64_t total_tokens,
                           int32_t heads, int64_t* keep_per_head) {
  if (!mean_diversity || !keep_per_head) return fail(KV_ERR_ARG, "mean_diversity or keep_per_head is NULL");
  if (n_layers < 1) return fail(KV_ERR_ARG, "n_layers must be >= 1");
  if (!(tau > 0.0) || !std::isfinite(tau)) return fail(KV_ERR_ARG, "tau must be finite and > 0");
  if (total_tokens < 0 || total_tokens > ((int64_t)1 << 53)) return fail(KV_ERR_ARG, "total_tokens out of range");
  if (heads < 1) return fail(KV_ERR_ARG, "heads must be >= 1");
  std::vector<double> z((size_t)n_layers);
  double mx = -INFINITY;
  for (int32_t i = 0; i < n_layers; ++i) {
    z[(size_t)i] = mean_diversity[i] / tau;
    if (!std::isfinite(z[(size_t)i])) return fail(KV_ERR_ARG, "mean_diversity[%d] / tau is not finite", i);
    mx = std::max(mx, z[(size_t)i]);
  }
  double sum = 0.0;
  for (auto& v : z) {
    v = std::exp(v - mx);
    sum += v;
  }
  for (int32_t i = 0; i < n_layers; ++i) {
    const double share = std::floor(z[(size_t)i] / sum * (double)total_tokens);
    keep_per_head[i] = (int64_t)std::floor(share / (double)heads);
  }
  return ok();
}

kv_status kv_get_head_lengths(const kv_pool_t* pool, int32_t layer, int32_t* lens, int32_t cap, int32_t* n_out) {
  kv_status s = check_layer(pool, layer);
  if (s != KV_OK) return s;
  if (cap < 0) return fail(KV_ERR_ARG, "negative cap");
  const auto& L = pool->layers[(size_t)layer];
  const int32_t n = (int32_t)L.table.size(), H = pool->cfg.num_heads;
  if (lens)
    for (int32_t i = 0; i < n && i < cap; ++i)
      for (int32_t h = 0; h < H; ++h) lens[(int64_t)i * H + h] = kvs::head_len(L.table[(size_t)i], h);
  if (n_out) *n_out = n;
  return ok();
}

kv_status kv_get_info(const kv_pool_t* pool, int32_t layer, kv_cache_info* out) {
  kv_status s = check_layer(pool, layer);
  if (s != KV_OK) return s;
  if (!out) return fail(KV_ERR_ARG, "out is NULL");
  const auto& L = pool->layers[(size_t)layer];
  out->persisted_frames = (int32_t)L.table.size() - L.special_pages();
  out->pages_used = (int32_t)L.table.size();
  out->pages_free = (int32_t)L.free_ids.size();
  out->transient_pending = L.transient_pending ? 1 : 0;
  out->tokens = L.tokens();
  out->bytes = (int64_t)L.table.size() * pool->lay.geom.page_bytes;
  out->evictions = L.evictions;
  out->compactions = L.compactions;
  out->last_keep_count = L.last_keep;
  out->merges = L.merges;
  out->prunes = L.prunes;
  out->special_pages = L.special_pages();
  out->special_tokens = L.special_tokens();
  return ok();
}

kv_status kv_get_page_table(const kv_pool_t* pool, int32_t layer, int32_t* page_ids, int32_t* page_lens,
                            int64_t* frame_ids, int32_t cap, int32_t* n_out) {
  kv_status s = check_layer(pool, layer);
  if (s != KV_OK) return s;
  if (cap < 0) return fail(KV_ERR_ARG, "negative cap");
  const auto& L = pool->layers[(size_t)layer];
  const int32_t n = (int32_t)L.table.size();
  for (int32_t i = 0; i < n && i < cap; ++i) {
    if (page_ids) page_ids[i] = L.table[(size_t)i].page;
    if (page_lens) page_lens[i] = L.table[(size_t)i].len;
    if (frame_ids) frame_ids[i] = L.table[(size_t)i].special ? -1 - L.table[(size_t)i].frame : L.table[(size_t)i].frame;
  }
  if (n_out) *n_out = n;
  return ok();
}

const char* kv_last_error(void) { return g_err.c_str(); }

}  // extern "C"
