// CLCES scoring, top-k keep and page-local compaction, gfx950.
//
// StreamCacheVGGT article, section 2.1: per window layer the N candidate
// tokens are ranked by raw score (2.1.1), the ranks are normalised to [0,1]
// and their mean / variance over the window give Cons = max(0, 1 -
// sigma*sqrt(12)) (2.1.2), fused as s_hat = s * (1 + lambda*Cons) (2.1.3).
// Top-k keep by s_hat and in-place compaction of the kept rows follow the
// article's "pure eviction" description (section 1) and the InfiniteVGGT
// explainer ("Rolling Memory", "Prune and roll the memory").
//
// Pipeline (one launch each, all on the caller's stream, one final sync):
//   prep     the page table (first chunk) and the counters set to zero;
//   gather   raw scores of every candidate at every window layer (by global
//            token id), validate them, write 32-bit order keys;
//   rank     stable LSD radix sort, 4 passes of 8 bits, all window layers at
//            once (histogram / scan / scatter; the scatter is made stable
//            with wave ballots); the last pass writes rank[token] directly;
//   fuse     float64 mean, population variance, Cons and s_hat with a fixed
//            operation order and no contraction (bit-exact reproducible),
//            plus the histogram of the first select digit;
//   select   radix select of the keep_count-th largest s_hat (8 passes of 8
//            bits over the 64-bit pattern, which orders non-negative doubles;
//            the first histogram comes from fuse, the last step from mark);
//   mark     per page: count of s_hat above / equal to the threshold;
//   index    per page: its kept count and offsets (from all pages' counts),
//            the kept token ids in slot order, and the moves: with
//            n kept, kept slots below n stay and the dropped slots below n
//            take the kept slots at or past n (both ascending);
//   compact  per page: one workgroup per K head, one per V head and one for
//            the token ids; sources (>= n) and destinations (< n) are
//            disjoint, so every row moves independently.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>
#include <cmath>
#include <utility>

#include "blockscan.h"
#include "clces.h"
#include "rowmove.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = kRankTile / kThreads;  // 2

struct SelState {
  unsigned long long prefix;
  long long k_rem;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

__device__ inline uint32_t order_key(float s) {
  const uint32_t b = __float_as_uint(s);
  return b == 0x80000000u ? 0u : b;  // -0.0 ranks as +0.0
}

// First launch of a step: the first page-table chunk, and the counters that
// later kernels accumulate into set to zero (the rank chunk sums of every
// pass, select histograms, per-page counts, the error flag).
__global__ void prep_kernel(DevEntry* entries, TableChunk chunk, uint32_t* rank_counts, int64_t n_rank,
                            uint32_t* sel_hist, int32_t* counts, int n_counts, int32_t* flag) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < chunk.count) entries[chunk.first + i] = chunk.e[i];
  if (i < n_rank) rank_counts[i] = 0;
  if (i < 8 * 256) sel_hist[i] = 0;
  if (i < n_counts) counts[i] = 0;
  if (i == 0) *flag = 0;
}

constexpr int kChunk = 16;  // rank blocks per chunk of the digit-offset scan

// Counts of one rank pass: [segment][block][digit] and the chunk sums
// [segment][chunk][digit].  The chunk sums of all 4 passes come first in the
// counter array (they accumulate with atomics, so only they are zeroed), then
// the block counts of all 4 passes (stored outright).
struct RankCounts {
  uint32_t* blk;
  uint32_t* chunk;
  int nblk, nchunk;
};

__host__ __device__ inline int64_t rank_chunk_counters(int segments, int nblk) {
  return 4 * (int64_t)segments * ((nblk + kChunk - 1) / kChunk) * 256;
}

__device__ inline RankCounts rank_counts(uint32_t* base, int pass, int segments, int nblk) {
  const int nchunk = (nblk + kChunk - 1) / kChunk;
  return RankCounts{base + rank_chunk_counters(segments, nblk) + (int64_t)pass * segments * nblk * 256,
                    base + (int64_t)pass * segments * nchunk * 256, nblk, nchunk};
}



struct GatherArgs {
  const DevEntry* entries;
  const char* pool;
  int64_t page_bytes, id_off;
  const float* table;
  int64_t rows;
  int32_t cols, first_layer, n_win, N;
  uint32_t* keys;  // [n_win][N]
  float* scur;     // [N]
  int32_t* flag;
};

__global__ __launch_bounds__(kThreads) void gather_kernel(GatherArgs g) {
  const DevEntry en = g.entries[blockIdx.x];
  const int j = blockIdx.y * kThreads + threadIdx.x;
  if (j >= en.len) return;
  const int32_t* ids = reinterpret_cast<const int32_t*>(g.pool + (int64_t)en.phys * g.page_bytes + g.id_off);
  const int32_t tok = ids[j];
  const int idx = en.tok_start + j;
  if (tok < 0 || (int64_t)tok >= g.rows) {
    atomicOr(g.flag, kClcesErrRow);
    return;
  }
  const float* row = g.table + (int64_t)tok * g.cols + g.first_layer;
  float s = 0.f;
  for (int w = 0; w < g.n_win; ++w) {
    s = row[w];
    if (!(s >= 0.f)) atomicOr(g.flag, kClcesErrNan);
    g.keys[(int64_t)w * g.N + idx] = order_key(s);
  }
  g.scur[idx] = __uint_as_float(order_key(s));
}

// Digit histogram of one block of one pass, counted in LDS (wave-aggregated:
// the top bytes of similar scores are nearly uniform), stored as the block's
// counts and added into its chunk's sums (at most kChunk workgroups add to
// one counter).
__global__ __launch_bounds__(kThreads) void rank_hist_kernel(const uint32_t* keys, uint32_t* counts, int N, int nblk,
                                                             int pass, const int32_t* flag) {
  if (*flag) return;
  __shared__ uint32_t cnt[256];
  const int w = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x, segments = gridDim.y;
  cnt[tid] = 0;
  __syncthreads();
  const uint32_t* k = keys + (int64_t)w * N;
  const int shift = 8 * pass;
  for (int j = 0; j < kItems; ++j) {
    const int i = blk * kRankTile + j * kThreads + tid;
    hist_add(cnt, i < N ? (k[i] >> shift) & 255u : 0u, i < N);
  }
  __syncthreads();
  const RankCounts rc = rank_counts(counts, pass, segments, nblk);
  rc.blk[((int64_t)w * nblk + blk) * 256 + tid] = cnt[tid];
  if (cnt[tid]) atomicAdd(&rc.chunk[((int64_t)w * rc.nchunk + blk / kChunk) * 256 + tid], cnt[tid]);
}

// One stable LSD pass over this block's kRankTile keys (kItems per thread;
// key i = blk*kRankTile + j*kThreads + tid, so index order is (item j, wave,
// lane)).  Every wave matches the digits of each of its items with ballots,
// giving each key its rank among equal digits of its (item, wave) group and
// each group's digit counts; one pass per digit then turns the counts into
// exclusive offsets in index order, and every key goes to
// offset[block][digit] + offset[group][digit] + rank.
__global__ __launch_bounds__(kThreads) void rank_scatter_kernel(const uint32_t* keys_in, const uint32_t* vals_in,
                                                                uint32_t* keys_out, uint32_t* vals_out,
                                                                int32_t* ranks, uint32_t* counts, int N,
                                                                int nblk, int pass, const int32_t* flag) {
  if (*flag) return;
  constexpr int kWaves = kThreads / 64;
  __shared__ uint32_t cnt[kItems][kWaves][256];
  const int w = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int segments = gridDim.y, shift = 8 * pass, last = pass == 3;
  __shared__ int32_t scan[kThreads];
  // where this block's keys of digit tid start in the segment: keys of smaller
  // digits in the whole segment (the chunk sums added over chunks, scanned
  // over digits), plus keys of digit tid in the chunks before this block's
  // chunk and in the blocks before it within its chunk
  uint32_t run;
  {
    const RankCounts rc = rank_counts(counts, pass, segments, nblk);
    const int c = blk / kChunk;
    const uint32_t* ct = rc.chunk + (int64_t)w * rc.nchunk * 256 + tid;
    uint32_t tot = 0, before = 0;
    for (int cc = 0; cc < rc.nchunk; ++cc) {
      const uint32_t x = ct[(int64_t)cc * 256];
      tot += x;
      before += cc < c ? x : 0u;
    }
    const uint32_t* col = rc.blk + ((int64_t)w * nblk + (int64_t)c * kChunk) * 256 + tid;
    for (int b = c * kChunk; b < blk; ++b) before += col[(int64_t)(b - c * kChunk) * 256];
    run = (uint32_t)block_excl_scan<kThreads>((int32_t)tot, scan, nullptr) + before;
  }
#pragma unroll
  for (int j = 0; j < kItems; ++j)
#pragma unroll
    for (int q = 0; q < kWaves; ++q) cnt[j][q][tid] = 0;
  const int64_t seg = (int64_t)w * N;
  const unsigned long long lt = (1ull << lane) - 1ull;
  uint32_t key[kItems], val[kItems], rnk[kItems];
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int i = blk * kRankTile + j * kThreads + tid;
    const bool valid = i < N;
    key[j] = valid ? keys_in[seg + i] : 0u;
    val[j] = valid ? (vals_in ? vals_in[seg + i] : (uint32_t)i) : 0u;
  }
  __syncthreads();  // counters zeroed
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int i = blk * kRankTile + j * kThreads + tid;
    const bool valid = i < N;
    const uint32_t d = (key[j] >> shift) & 255u;
    unsigned long long m = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (d >> bit) & 1u;
      const unsigned long long bb = __ballot(on);
      m &= on ? bb : ~bb;
    }
    rnk[j] = (uint32_t)__popcll(m & lt);
    if (valid && rnk[j] == 0) cnt[j][wave][d] = (uint32_t)__popcll(m);
  }
  __syncthreads();
  // thread tid owns digit tid: exclusive offsets over the groups in index order
#pragma unroll
  for (int j = 0; j < kItems; ++j)
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
      const uint32_t c = cnt[j][q][tid];
      cnt[j][q][tid] = run;
      run += c;
    }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int i = blk * kRankTile + j * kThreads + tid;
    if (i < N) {
      const uint32_t d = (key[j] >> shift) & 255u;
      const uint32_t off = cnt[j][wave][d] + rnk[j];
      if (last) {
        ranks[seg + val[j]] = (int32_t)off;
      } else {
        keys_out[seg + off] = key[j];
        vals_out[seg + off] = val[j];
      }
    }
  }
}

// Also the first select pass: the histogram of the top byte of s_hat, and
// the state before it (nothing fixed, keep_count to find).
__global__ __launch_bounds__(kThreads) void fuse_kernel(const int32_t* ranks, const float* scur,
                                                        unsigned long long* shat, int N, int n_win, double lambda,
                                                        double sqrt12, uint32_t* sel_hist, SelState* states,
                                                        long long keep, const int32_t* flag) {
#pragma clang fp contract(off)
  if (*flag) return;
  __shared__ uint32_t cnt[256];
  cnt[threadIdx.x] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) states[0] = SelState{0ull, keep};
  __syncthreads();
  const int i = blockIdx.x * kThreads + threadIdx.x;
  const bool valid = i < N;
  unsigned long long bits = 0;
  if (valid) {
  const double denom = (double)(N - 1);
  double r[8];
  double acc = 0.0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    if (w < n_win) {
      r[w] = N > 1 ? (double)ranks[(int64_t)w * N + i] / denom : 0.0;
      acc = acc + r[w];
    }
  }
  const double mu = acc / (double)n_win;
  double acc2 = 0.0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    if (w < n_win) {
      const double d = r[w] - mu;
      acc2 = acc2 + d * d;
    }
  }
  const double var = acc2 / (double)n_win;
  const double sigma = sqrt(var);
  const double c = 1.0 - sigma * sqrt12;
  const double cons = c > 0.0 ? c : 0.0;
  const double sh = (double)scur[i] * (1.0 + lambda * cons) + 0.0;
  bits = (unsigned long long)__double_as_longlong(sh);
  shat[i] = bits;
  }
  hist_add(cnt, (uint32_t)(bits >> 56), valid);
  __syncthreads();
  if (cnt[threadIdx.x]) atomicAdd(&sel_hist[threadIdx.x], cnt[threadIdx.x]);
}

// One select step: from the state before pass p and that pass's digit
// histogram, fix digit p (the largest digit whose suffix count reaches k_rem)
// and reduce k_rem by the count of larger digits.  Wave 0 runs a suffix scan
// over its 64 lanes (4 digits each); the result is broadcast through LDS.
__device__ SelState select_advance(SelState st, const uint32_t* hist, int p) {
  __shared__ uint32_t cnt[256];
  __shared__ SelState out;
  cnt[threadIdx.x] = hist[threadIdx.x];
  if (threadIdx.x == 0) out = st;
  __syncthreads();
  if (threadIdx.x < 64 && st.k_rem > 0) {
    const int lane = threadIdx.x;
    long long own = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) own += cnt[4 * lane + j];
    long long suf = own;  // inclusive suffix sum over lanes >= lane
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long t = __shfl_down(suf, off, 64);
      if (lane + off < 64) suf += t;
    }
    long long above = __shfl_down(suf, 1, 64);  // lanes > lane
    if (lane == 63) above = 0;
    if (above < st.k_rem && suf >= st.k_rem) {
      long long cum = above;
      for (int j = 3; j >= 0; --j) {
        const long long c = cnt[4 * lane + j];
        if (cum + c >= st.k_rem) {
          out.prefix = st.prefix | ((unsigned long long)(4 * lane + j) << (56 - 8 * p));
          out.k_rem = st.k_rem - cum;
          break;
        }
        cum += c;
      }
    }
  }
  __syncthreads();
  const SelState r = out;
  __syncthreads();
  return r;
}

// Pass p histograms digit p of the keys that match the digits fixed so far.
// The state before pass p is advanced once from the previous pass's state
// (stored by its workgroup 0) and histogram; workgroup 0 stores it in turn.
__global__ __launch_bounds__(kThreads) void select_pass_kernel(const unsigned long long* keys, int N,
                                                               uint32_t* sel_hist, SelState* states, long long keep,
                                                               int p, const int32_t* flag) {
  if (*flag) return;
  __shared__ uint32_t cnt[256];
  const SelState st = p == 0 ? SelState{0ull, keep} : select_advance(states[p - 1], sel_hist + (p - 1) * 256, p - 1);
  if (blockIdx.x == 0 && threadIdx.x == 0) states[p] = st;
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int shift = 56 - 8 * p;
  const unsigned long long hi = p == 0 ? 0ull : (~0ull << (shift + 8));
  for (int j = 0; j < kItems; ++j) {
    const int i = blockIdx.x * kRankTile + j * kThreads + threadIdx.x;
    const unsigned long long k = i < N ? keys[i] : 0ull;
    const bool match = i < N && (k & hi) == st.prefix;
    hist_add(cnt, (uint32_t)((k >> shift) & 255ull), match);
  }
  __syncthreads();
  if (cnt[threadIdx.x]) atomicAdd(&sel_hist[p * 256 + threadIdx.x], cnt[threadIdx.x]);
}

struct MarkArgs {
  const DevEntry* entries;
  const unsigned long long* shat;
  const uint32_t* sel_hist;
  long long keep;
  int32_t* n_gt;
  int32_t* n_eq;
  SelState* states;  // [0..7] states before each pass, [8] the final threshold
  const int32_t* flag;
};

__global__ __launch_bounds__(kThreads) void mark_kernel(MarkArgs a) {
  if (*a.flag) return;
  __shared__ int32_t sg, se;
  // threshold = the keep_count-th largest key; keep 0 keeps nothing
  SelState st = a.keep == 0 ? SelState{~0ull, 0} : select_advance(a.states[7], a.sel_hist + 7 * 256, 7);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) a.states[8] = st;
  if (threadIdx.x == 0) { sg = 0; se = 0; }
  __syncthreads();
  const DevEntry en = a.entries[blockIdx.x];
  const int j = blockIdx.y * kThreads + threadIdx.x;
  int gt = 0, eq = 0;
  if (j < en.len) {
    const unsigned long long k = a.shat[en.tok_start + j];
    gt = k > st.prefix;
    eq = k == st.prefix;
  }
  const unsigned long long bg = __ballot(gt), be = __ballot(eq);
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(&sg, (int32_t)__popcll(bg));
    atomicAdd(&se, (int32_t)__popcll(be));
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (sg) atomicAdd(&a.n_gt[blockIdx.x], sg);
    if (se) atomicAdd(&a.n_eq[blockIdx.x], se);
  }
}

struct CompactArgs {
  const DevEntry* entries;
  uint16_t* move_src;    // [P][ts] kept slots at or past the new length, ascending
  uint16_t* move_dst;    // [P][ts] dropped slots below the new length, ascending
  int32_t* n_moves;      // [P]
  const unsigned long long* shat;
  const SelState* final_state;
  const int32_t* n_gt;   // [P] keys above the threshold, per page
  const int32_t* n_eq;   // [P] keys equal to the threshold, per page
  int32_t* new_len;      // [P] written here: kept slots per page
  int32_t n_entries;
  char* pool;
  PageGeom g;
  int32_t* keep_ids_out;
  const int32_t* flag;
  int32_t* flag_rw;
};

// Per page: which slots are kept (ties at the threshold in index order, from
// the plan step's tie rank base), the kept token ids in slot order, and the
// moves of the compaction.  With n = new length, kept slots below n stay; the
// dropped slots below n (the holes, ascending) take the kept slots at or past
// n (ascending).  Sources and destinations are disjoint, so the moves can run
// in any order.
__global__ __launch_bounds__(kThreads) void index_kernel(CompactArgs a) {
  if (*a.flag) return;
  __shared__ int32_t scan[kThreads];
  __shared__ uint16_t kept[kMaxPageTokensScored];
  const int e = blockIdx.x, tid = threadIdx.x;
  const DevEntry en = a.entries[e];
  const int len = en.len;
  const SelState st = *a.final_state;
  // This page's plan.  Keys equal to the threshold are kept in index order
  // until k_rem of them are, so the pages before this one keep
  // sum(n_gt) + min(k_rem, sum(n_eq)) keys, and this page's ties are ranked
  // from sum(n_eq) over those pages.
  int32_t gt_before = 0, eq_before = 0;
  for (int i = tid; i < e; i += kThreads) {
    gt_before += a.n_gt[i];
    eq_before += a.n_eq[i];
  }
  int32_t gt_tot = 0, eq_tot = 0;
  block_excl_scan<kThreads>(gt_before, scan, &gt_tot);
  block_excl_scan<kThreads>(eq_before, scan, &eq_tot);
  const long long k_rem = st.k_rem;
  const long long eq_take = k_rem - eq_tot;
  const int32_t nl = a.n_gt[e] + (int32_t)(eq_take < 0 ? 0 : (eq_take > a.n_eq[e] ? a.n_eq[e] : eq_take));
  const int32_t keep_base = gt_tot + (int32_t)(k_rem < eq_tot ? (k_rem < 0 ? 0 : k_rem) : eq_tot);
  if (tid == 0) a.new_len[e] = nl;
  const int per = (len + kThreads - 1) / kThreads;
  const int b = tid * per, end = min(b + per, len);
  const unsigned long long* sh = a.shat + en.tok_start;
  int32_t n_eq = 0;
  for (int j = b; j < end; ++j) n_eq += sh[j] == st.prefix;
  const int32_t eq_start = eq_tot + block_excl_scan<kThreads>(n_eq, scan, nullptr);
  int32_t eq_rank = eq_start;
  int32_t n_keep = 0, n_hole = 0;
  for (int j = b; j < end; ++j) {
    const unsigned long long k = sh[j];
    bool keep = k > st.prefix;
    if (k == st.prefix) keep = eq_rank++ < st.k_rem;
    n_keep += keep;
    n_hole += !keep && j < nl;
  }
  int32_t kept_total = 0, holes = 0;
  int32_t pos = block_excl_scan<kThreads>(n_keep, scan, &kept_total);
  int32_t hpos = block_excl_scan<kThreads>(n_hole, scan, &holes);
  if (kept_total != nl) {  // cannot happen when the plan and this pass agree; never move on a mismatch
    if (tid == 0) {
      atomicOr(a.flag_rw, kClcesErrCount);
      a.n_moves[e] = 0;
    }
    return;
  }
  uint16_t* dst = a.move_dst + (int64_t)e * a.g.ts;
  eq_rank = eq_start;
  for (int j = b; j < end; ++j) {
    const unsigned long long k = sh[j];
    bool keep = k > st.prefix;
    if (k == st.prefix) keep = eq_rank++ < st.k_rem;
    if (keep)
      kept[pos++] = (uint16_t)j;
    else if (j < nl)
      dst[hpos++] = (uint16_t)j;
  }
  __syncthreads();
  // fillers: the kept slots at or past nl are the last `holes` entries of the kept list
  uint16_t* src = a.move_src + (int64_t)e * a.g.ts;
  for (int k = tid; k < holes; k += kThreads) src[k] = kept[nl - holes + k];
  if (a.keep_ids_out) {
    const int32_t* ids = reinterpret_cast<const int32_t*>(a.pool + (int64_t)en.phys * a.g.page_bytes + a.g.id_off);
    for (int i = tid; i < nl; i += kThreads) a.keep_ids_out[keep_base + i] = ids[kept[i]];
  }
  if (tid == 0) a.n_moves[e] = holes;
}


// Grid (page, part): part < H moves the K rows of head `part`, H <= part < 2H
// the V rows of head part - H, part 2H the token ids.
template <typename T, int NT>
__global__ __launch_bounds__(NT) void compact_kernel(CompactArgs a) {
  if (*a.flag) return;
  const int e = blockIdx.x, part = blockIdx.y, tid = threadIdx.x;
  const int nm = a.n_moves[e];
  if (nm == 0) return;
  const int H = a.g.heads;
  const DevEntry en = a.entries[e];
  const uint16_t* src = a.move_src + (int64_t)e * a.g.ts;
  const uint16_t* dst = a.move_dst + (int64_t)e * a.g.ts;
  char* page = a.pool + (int64_t)en.phys * a.g.page_bytes;
  if (part < 2 * H) {
    constexpr int VPR = 64 * sizeof(T) / 16;
    const int h = part < H ? part : part - H;
    V16* rows = reinterpret_cast<V16*>(page + (part < H ? a.g.k_off : a.g.v_off)) + (int64_t)h * a.g.ts * VPR;
    move_rows<T, NT>(rows, src, dst, nm, tid);
  } else {
    int32_t* ids = reinterpret_cast<int32_t*>(page + a.g.id_off);
    for (int i = tid; i < nm; i += NT) ids[dst[i]] = ids[src[i]];
  }
}

}  // namespace

ClcesSizes clces_sizes(int64_t n_max, int32_t p_max, int32_t w_max, int32_t ts_max) {
  ClcesSizes z{};
  z.n_max = n_max;
  z.p_max = p_max;
  z.w_max = w_max;
  z.nblk_max = (int32_t)((n_max + kRankTile - 1) / kRankTile);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t wn = (size_t)w_max * (size_t)n_max;
  z.keys_a = take(wn * 4);
  z.keys_b = take(wn * 4);
  z.vals_a = take(wn * 4);
  z.vals_b = take(wn * 4);
  z.ranks = take(wn * 4);
  z.scur = take((size_t)n_max * 4);
  z.shat = take((size_t)n_max * 8);
  z.hist = take((size_t)rank_counters((int)n_max, w_max) * 4);  // rank counts of the 4 passes
  z.sel_hist = take(8 * 256 * 4);
  z.sel_state = take(9 * sizeof(SelState));
  z.entries = take((size_t)p_max * sizeof(DevEntry));
  z.counts = take((size_t)p_max * 2 * 4);
  z.move_src = take((size_t)p_max * ts_max * 2);
  z.move_dst = take((size_t)p_max * ts_max * 2);
  z.n_moves = take((size_t)p_max * 4);
  z.flag = take(((size_t)p_max + 1) * 4);  // the error flag, then the new page lengths [p_max]
  z.total = off;
  return z;
}

int64_t rank_counters(int N, int segments) {
  const int nblk = (N + kRankTile - 1) / kRankTile;
  return rank_chunk_counters(segments, nblk) + 4 * (int64_t)segments * nblk * 256;
}

hipError_t launch_rank_segments(uint32_t* keys_a, uint32_t* keys_b, uint32_t* vals_a, uint32_t* vals_b, int32_t* ranks,
                                uint32_t* counts, int N, int segments, const int32_t* flag, hipStream_t s) {
  const int nblk = (N + kRankTile - 1) / kRankTile;
  uint32_t* kin = keys_a;
  uint32_t* kout = keys_b;
  uint32_t* vin = nullptr;
  uint32_t* vout = vals_b;
  for (int pass = 0; pass < 4; ++pass) {
    rank_hist_kernel<<<dim3((unsigned)nblk, (unsigned)segments), dim3(kThreads), 0, s>>>(kin, counts, N, nblk, pass,
                                                                                          flag);
    rank_scatter_kernel<<<dim3((unsigned)nblk, (unsigned)segments), dim3(kThreads), 0, s>>>(
        kin, vin, kout, vout, ranks, counts, N, nblk, pass, flag);
    std::swap(kin, kout);
    vin = vout;
    vout = vout == vals_b ? vals_a : vals_b;
  }
  return hipGetLastError();
}

hipError_t enqueue_clces(const ClcesArgs& a, hipStream_t s) {
  const ClcesSizes& z = a.sizes;
  char* ws = a.ws;
  auto* entries = reinterpret_cast<DevEntry*>(ws + z.entries);
  auto* keys_a = reinterpret_cast<uint32_t*>(ws + z.keys_a);
  auto* keys_b = reinterpret_cast<uint32_t*>(ws + z.keys_b);
  auto* vals_a = reinterpret_cast<uint32_t*>(ws + z.vals_a);
  auto* vals_b = reinterpret_cast<uint32_t*>(ws + z.vals_b);
  auto* ranks = a.ranks_out ? a.ranks_out : reinterpret_cast<int32_t*>(ws + z.ranks);
  auto* scur = reinterpret_cast<float*>(ws + z.scur);
  auto* shat = reinterpret_cast<unsigned long long*>(ws + z.shat);
  auto* hist = reinterpret_cast<uint32_t*>(ws + z.hist);
  auto* sel_hist = reinterpret_cast<uint32_t*>(ws + z.sel_hist);
  auto* sel_state = reinterpret_cast<SelState*>(ws + z.sel_state);
  auto* counts = reinterpret_cast<int32_t*>(ws + z.counts);
  auto* flag = reinterpret_cast<int32_t*>(ws + z.flag);
  const int P = a.n_entries, N = a.n_tokens, W = a.n_window;
  if (P > z.p_max || (int64_t)N > z.n_max || W > z.w_max || a.geom.ts > kMaxPageTokensScored)
    return hipErrorInvalidValue;

  {
    TableChunk c;
    c.first = 0;
    c.count = std::min(P, kUploadChunk);
    for (int i = 0; i < c.count; ++i) c.e[i] = a.entries_host[i];
    const int64_t n_rank = rank_chunk_counters(W, (N + kRankTile - 1) / kRankTile);  // the chunk sums
    const int64_t nz = std::max<int64_t>(std::max(8 * 256, 2 * P), n_rank);
    prep_kernel<<<dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, s>>>(entries, c, hist, n_rank, sel_hist, counts,
                                                                          2 * P, flag);
  }
  hipError_t e = P > kUploadChunk ? launch_table_upload(entries + kUploadChunk, a.entries_host + kUploadChunk,
                                                        P - kUploadChunk, s)
                                  : hipGetLastError();
  if (e != hipSuccess) return e;

  GatherArgs g{entries, a.pool, a.geom.page_bytes, a.geom.id_off, a.score_table, a.score_rows, a.score_cols,
               a.first_layer, W, N, keys_a, scur, flag};
  gather_kernel<<<dim3((unsigned)P, (unsigned)((a.geom.ts + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(g);

  const int nblk = (N + kRankTile - 1) / kRankTile;
  e = launch_rank_segments(keys_a, keys_b, vals_a, vals_b, ranks, hist, N, W, flag, s);
  if (e != hipSuccess) return e;
  fuse_kernel<<<dim3((unsigned)((N + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(
      ranks, scur, shat, N, W, a.lambda, std::sqrt(12.0), sel_hist, sel_state, a.keep, flag);
  if (a.keep > 0) {
    for (int p = 1; p < 8; ++p)
      select_pass_kernel<<<dim3((unsigned)nblk), dim3(kThreads), 0, s>>>(shat, N, sel_hist, sel_state, a.keep, p,
                                                                         flag);
  }
  MarkArgs m{entries, shat, sel_hist, a.keep, counts, counts + P, sel_state, flag};
  mark_kernel<<<dim3((unsigned)P, (unsigned)((a.geom.ts + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(m);
  CompactArgs ca{entries,
                 reinterpret_cast<uint16_t*>(ws + z.move_src),
                 reinterpret_cast<uint16_t*>(ws + z.move_dst),
                 reinterpret_cast<int32_t*>(ws + z.n_moves),
                 shat, sel_state + 8, counts, counts + P, flag + 1, P, a.pool, a.geom, a.keep_ids_out, flag,
                 flag};
  index_kernel<<<dim3((unsigned)P), dim3(kThreads), 0, s>>>(ca);
  dim3 cg((unsigned)P, (unsigned)(2 * a.geom.heads + 1));
  const bool many = (int64_t)(N - a.keep) * 10 > (int64_t)N;  // more than 10% of the tokens drop
  if (a.geom.esize == 2) {
    if (many)
      compact_kernel<__bf16, 1024><<<cg, dim3(1024), 0, s>>>(ca);
    else
      compact_kernel<__bf16, 256><<<cg, dim3(256), 0, s>>>(ca);
  } else {
    if (many)
      compact_kernel<float, 1024><<<cg, dim3(1024), 0, s>>>(ca);
    else
      compact_kernel<float, 256><<<cg, dim3(256), 0, s>>>(ca);
  }
  return hipGetLastError();
}

int32_t* clces_result(const ClcesArgs& a) { return reinterpret_cast<int32_t*>(a.ws + a.sizes.flag); }

hipError_t run_clces(const ClcesArgs& a, int32_t* new_lens_host, int32_t* err_flag_host, hipStream_t s) {
  hipError_t e = enqueue_clces(a, s);
  if (e != hipSuccess) return e;
  // one read-back: the error flag and, after it, the new page lengths
  std::vector<int32_t> rb((size_t)a.n_entries + 1);
  e = hipMemcpyAsync(rb.data(), clces_result(a), sizeof(int32_t) * rb.size(), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  *err_flag_host = rb[0];
  std::copy(rb.begin() + 1, rb.end(), new_lens_host);
  return hipSuccess;
}

}  // namespace kvs
