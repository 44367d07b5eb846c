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
//   gather   raw scores of every candidate at every window layer whose ranks
//            are not reused from an earlier step (by global token id),
//            validate them, write 32-bit order keys;
//   rank     stable ranks of those layers' keys: every block of 2048 keys
//            sorted in LDS (each key's rank within its block), then each
//            key's count of smaller keys in the other blocks by binary search,
//            per group of blocks (two launches); or, where segments x blocks^2
//            is large, 4 LSD radix passes of 8 bits over the blocks (eight);
//   fuse     the ranks as the sums of those counts (stored for later steps),
//            float64 mean, population variance, Cons and s_hat with a fixed
//            operation order and no contraction (bit-exact reproducible),
//            plus the histogram of the first select digit;
//   select   radix select of the keep_count-th largest s_hat (up to 6
//            passes of 11, 11, 11, 11, 11 and 9 bits over the 64-bit
//            pattern, which orders non-negative doubles): the first histogram
//            comes from fuse, the second from a pass over every key, and one
//            workgroup finishes from there (the first 22 bits almost always
//            decide; otherwise it copies the still-matching keys to LDS);
//   mark     per page: count of s_hat above / equal to the threshold;
//   index    per page: its kept count and offsets (from all pages' counts),
//            the kept token ids in slot order, and the moves: with
//            n kept, kept slots below n stay and the dropped slots below n
//            take the kept slots at or past n (both ascending); a waiting
//            host may take each page's new length from a word in mapped host
//            memory that this step writes;
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
constexpr int kItems = 2;                      // keys per thread of the select passes
constexpr int kSelTile = kThreads * kItems;    // keys per select workgroup
constexpr int kSelBins = 1 << kSelBits;        // bins of a select digit

// Select state: the key bits fixed so far (prefix, under mask) and how many
// of the keys matching them are still to be kept.  done: no later pass can
// change the outcome (every matching key is kept, or nothing is to be kept,
// or all bits are fixed), so later passes only pass the state on.
struct SelState {
  unsigned long long prefix;
  unsigned long long mask;
  long long k_rem;
  int32_t done;
  int32_t match;  // keys matching the prefix (set by each advance; 0 before pass 0)
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

__device__ inline uint32_t order_key(float s) {
  const uint32_t b = __float_as_uint(s);
  return b == 0x80000000u ? 0u : b;  // -0.0 ranks as +0.0
}

// First launch of a step: the first page-table chunk, and the counters that
// later kernels accumulate into set to zero (select histograms, per-page
// counts, the error flag).
__global__ void prep_kernel(DevEntry* entries, TableChunk chunk, uint32_t* sel_hist, int n_hist, int32_t* counts,
                            int n_counts, int32_t* list_cnt, int32_t* flag) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < chunk.count) entries[chunk.first + i] = chunk.e[i];
  if (i < n_hist) sel_hist[i] = 0;
  if (i < n_counts) counts[i] = 0;
  if (i == 0) {
    *flag = 0;
    *list_cnt = 0;
  }
}

struct GatherArgs {
  const DevEntry* entries;
  const char* pool;
  int64_t page_bytes, id_off;
  const float* table;
  int64_t rows;
  int32_t cols, col_cur, n_seg, N;
  int32_t seg_col[kMaxWindow];  // score-table column of each segment to rank
  uint32_t* keys;  // [n_seg][N]
  float* scur;     // [N] the current layer's raw score
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
  const float* row = g.table + (int64_t)tok * g.cols;
  bool bad = false;
  for (int w = 0; w < g.n_seg; ++w) {
    const float s = row[g.seg_col[w]];
    bad = bad || !(s >= 0.f);
    g.keys[(int64_t)w * g.N + idx] = order_key(s);
  }
  const float s = row[g.col_cur];
  bad = bad || !(s >= 0.f);
  if (bad) atomicOr(g.flag, kClcesErrNan);
  g.scur[idx] = __uint_as_float(order_key(s));
}

// Stable rank of every key of a segment: the number of keys that are smaller,
// or equal at a smaller index.  Split by blocks of kRankTile consecutive
// indices, that is, for a key in block a, its rank within a plus, per other
// block b, the count of b's keys below it (b after a) or at most it (b before
// a).  Two launches:
//   rank_sort_kernel   one workgroup per block: a stable LSD radix sort of the
//                      block in LDS (4 passes of 8 bits; within each wave the
//                      keys of equal digit are matched with ballots, giving
//                      each key its rank among equal digits of its (item,
//                      wave) group and each group's digit counts; a pass over
//                      the groups in index order turns those into offsets).
//                      It writes the block's sorted keys, the index of each,
//                      and each key's rank within the block (count slice 0);
//   rank_count_kernel  one workgroup per (block a, group g of blocks): the
//                      sorted keys of group g's blocks in LDS, and the count
//                      of each of a's keys in every block of g but a (count
//                      slice 1 + g) by binary search.
// The rank is the sum of the slices, taken where it is used (fuse_kernel).
constexpr int kRankThreads = 1024;
constexpr int kRankItems = kRankTile / kRankThreads;  // 2
constexpr int kRankWaves = kRankThreads / 64;
constexpr int kRankGroupsIdx = kRankItems * kRankWaves;  // (item, wave) groups of a block
constexpr int kCountThreads = 256;
constexpr int kCountItems = kRankTile / kCountThreads;  // 8
constexpr int kCountChunk = 8;                           // blocks in LDS at once (64 KB)
constexpr uint32_t kPadKey = 0xFFFFFFFFu;  // above every valid key (those have the sign bit clear)

// Exclusive prefix over the 256 digits: thread d (< 256) passes digit d's
// count and gets the counts of digits below d (threads past 255 pass 0 and
// get nothing useful).  Every thread of the workgroup calls it.
__device__ inline uint32_t digit_excl_scan(uint32_t v, uint32_t* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(x, off, 64);
    if (lane >= off) x += t;
  }
  if (wave < 4 && lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t add = 0;
  for (int q = 0; q < wave && q < 4; ++q) add += wsum[q];
  return x - v + add;
}

// sorted, sorted_idx: [segments][Ns], Ns = whole blocks (kRankTile-aligned)
__global__ __launch_bounds__(kRankThreads) void rank_sort_kernel(const uint32_t* keys, uint32_t* sorted,
                                                                 uint32_t* sorted_idx, int32_t* part, int N,
                                                                 int64_t Ns, const int32_t* flag) {
  if (*flag) return;
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t cnt[kRankGroupsIdx][256];
  __shared__ uint32_t kbuf[kRankTile];
  __shared__ uint16_t ibuf[kRankTile];
  const int blk = blockIdx.x, w = blockIdx.y, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int start = blk * kRankTile;
  const int n = min(kRankTile, N - start);
  const int64_t seg = (int64_t)w * N;
  const int64_t sseg = (int64_t)w * Ns;
  // item j of thread tid is the key at block position j*kRankThreads + tid
  // (index order: item, wave, lane); positions past n hold the pad key, which
  // sorts after every valid key
  uint32_t key[kRankItems], idx[kRankItems];
#pragma unroll
  for (int j = 0; j < kRankItems; ++j) {
    const int p = j * kRankThreads + tid;
    key[j] = p < n ? keys[seg + start + p] : kPadKey;
    idx[j] = (uint32_t)p;
  }
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 8 * pass;
    for (int x = tid; x < kRankGroupsIdx * 256; x += kRankThreads) (&cnt[0][0])[x] = 0;
    __syncthreads();  // counters zeroed; the previous pass's reads of kbuf and ibuf are done
    uint32_t d[kRankItems], rnk[kRankItems];
#pragma unroll
    for (int j = 0; j < kRankItems; ++j) {
      d[j] = (key[j] >> shift) & 255u;
      unsigned long long m = ~0ull;
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const bool on = (d[j] >> bit) & 1u;
        const unsigned long long bb = __ballot(on);
        m &= on ? bb : ~bb;
      }
      rnk[j] = (uint32_t)__popcll(m & lt);
      if (rnk[j] == 0) cnt[j * kRankWaves + wave][d[j]] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    // thread t < 256 owns digit t: its offset is the count of smaller digits,
    // then the counts of the groups before it in index order
    uint32_t c[kRankGroupsIdx];
    uint32_t total = 0;
    if (tid < 256) {
#pragma unroll
      for (int q = 0; q < kRankGroupsIdx; ++q) {
        c[q] = cnt[q][tid];
        total += c[q];
      }
    }
    const uint32_t base = digit_excl_scan(tid < 256 ? total : 0u, wsum);
    if (tid < 256) {
      uint32_t run = base;
#pragma unroll
      for (int q = 0; q < kRankGroupsIdx; ++q) {
        cnt[q][tid] = run;
        run += c[q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRankItems; ++j) {
      const uint32_t np = cnt[j * kRankWaves + wave][d[j]] + rnk[j];
      kbuf[np] = key[j];
      ibuf[np] = (uint16_t)idx[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRankItems; ++j) {
      const int p = j * kRankThreads + tid;
      key[j] = kbuf[p];
      idx[j] = ibuf[p];
    }
  }
  // sorted position r: the pad keys are last, so r < n holds every valid key;
  // the whole block is written, pads included
#pragma unroll
  for (int j = 0; j < kRankItems; ++j) {
    const int r = j * kRankThreads + tid;
    sorted[sseg + start + r] = key[j];
    if (r < n) {
      sorted_idx[sseg + start + r] = idx[j];
      part[(int64_t)w * kRankParts * N + start + idx[j]] = r;
    }
  }
}

// The multi-pass alternative (taken where segments x blocks^2 grows large,
// since the counts above cost N x blocks searches): a stable LSD radix sort of
// the keys, 4 passes of 8 bits over the same blocks, two launches each:
//   rank_hist_kernel     the digit counts of each block, stored as they are;
//   rank_scatter_kernel  thread d < 256 adds digit d's counts over every block
//                        of the segment (total) and over the blocks before
//                        its own (before), all loads in flight together; the
//                        keys of digit d go to (keys of smaller digits) +
//                        (keys of digit d in earlier blocks) + (their rank in
//                        this block), ranked within the block by the same
//                        ballot matching; the last pass writes each key's rank.
constexpr int kHistThreads = 256;
struct RankOut {
  int32_t* seg[kMaxWindow];
};

__global__ __launch_bounds__(kHistThreads) void rank_hist_kernel(const uint32_t* keys, uint32_t* blk_cnt, int N,
                                                                 int nblk, int pass, const int32_t* flag) {
  if (*flag) return;
  __shared__ uint32_t cnt[256];
  const int w = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  const uint32_t* k = keys + (int64_t)w * N;
  const int shift = 8 * pass;
  constexpr int kPer = kRankTile / kHistThreads;  // 8
  uint32_t d[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = blk * kRankTile + j * kHistThreads + tid;
    d[j] = i < N ? (k[i] >> shift) & 255u : 0u;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) hist_add(cnt, d[j], blk * kRankTile + j * kHistThreads + tid < N);
  __syncthreads();
  blk_cnt[((int64_t)w * nblk + blk) * 256 + tid] = cnt[tid];
}

__global__ __launch_bounds__(kRankThreads) void rank_scatter_kernel(const uint32_t* keys_in, const uint32_t* vals_in,
                                                                    uint32_t* keys_out, uint32_t* vals_out,
                                                                    const uint32_t* blk_cnt, RankOut out, int N,
                                                                    int nblk, int pass, const int32_t* flag) {
  if (*flag) return;
  __shared__ uint32_t wsum[4];
  __shared__ uint32_t cnt[kRankItems][kRankWaves][256];
  __shared__ uint32_t part[2][4][256];
  const int w = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int shift = 8 * pass, last = pass == 3;
  const int64_t seg = (int64_t)w * N;
#pragma unroll
  for (int j = 0; j < kRankItems; ++j)
    for (int q = tid >> 8; q < kRankWaves; q += kRankThreads / 256) cnt[j][q][tid & 255] = 0;
  // digit d's counts over the segment and over the blocks before this one:
  // four threads per digit, each adding every fourth block with all its loads
  // in flight together, then combined through LDS
  {
    const int d = tid & 255, q = tid >> 8;
    const uint32_t* col = blk_cnt + (int64_t)w * nblk * 256 + d;
    constexpr int kBatch = 16;  // blocks per thread and batch: 64 blocks (131,072 keys) in one batch
    uint32_t b = 0, t = 0;
    for (int c0 = 0; c0 < nblk; c0 += 4 * kBatch) {
      uint32_t x[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int c = c0 + 4 * j + q;
        x[j] = c < nblk ? col[(int64_t)c * 256] : 0u;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        t += x[j];
        b += c0 + 4 * j + q < blk ? x[j] : 0u;
      }
    }
    part[0][q][d] = b;
    part[1][q][d] = t;
  }
  const int start = blk * kRankTile;
  const uint32_t* ks = keys_in + seg;
  uint32_t key[kRankItems], val[kRankItems], rnk[kRankItems];
  const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
  for (int j = 0; j < kRankItems; ++j) {
    const int i = start + j * kRankThreads + tid;
    const bool valid = i < N;
    key[j] = valid ? ks[i] : 0u;
    val[j] = valid ? (vals_in ? vals_in[seg + i] : (uint32_t)i) : 0u;
  }
  __syncthreads();  // counters zeroed
#pragma unroll
  for (int j = 0; j < kRankItems; ++j) {
    const bool valid = start + j * kRankThreads + tid < N;
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
  // thread d < 256 owns digit d: exclusive offsets over the groups in index order
  uint32_t before = 0, total = 0;
  if (tid < 256) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      before += part[0][q][tid];
      total += part[1][q][tid];
    }
  }
  const uint32_t base = digit_excl_scan(tid < 256 ? total : 0u, wsum);  // its barrier also orders cnt
  if (tid < 256) {
    uint32_t run = base + before;
#pragma unroll
    for (int j = 0; j < kRankItems; ++j)
#pragma unroll
      for (int q = 0; q < kRankWaves; ++q) {
        const uint32_t c = cnt[j][q][tid];
        cnt[j][q][tid] = run;
        run += c;
      }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kRankItems; ++j) {
    const int i = start + j * kRankThreads + tid;
    if (i < N) {
      const uint32_t d = (key[j] >> shift) & 255u;
      const uint32_t off = cnt[j][wave][d] + rnk[j];
      if (last) {
        out.seg[w][val[j]] = (int32_t)off;
      } else {
        keys_out[seg + off] = key[j];
        vals_out[seg + off] = val[j];
      }
    }
  }
}

// tab: dynamic LDS of min(largest group, kCountChunk) blocks.  Lanes take
// consecutive sorted keys of block a (key r = j*kCountThreads + thread), so
// the lanes of a wave follow nearly the same path down each search (broadcast
// reads first, then neighbouring words).  Each key's count in a block is a
// binary search over byte offsets (the step goes into the read's offset),
// eight keys per thread in flight together.
__global__ __launch_bounds__(kCountThreads) void rank_count_kernel(const uint32_t* sorted, const uint32_t* sorted_idx,
                                                                   int32_t* part, int N, int64_t Ns, int nblk,
                                                                   int groups, int chunk, const int32_t* flag) {
  if (*flag) return;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  constexpr int kVec = kRankTile / 4 / kCountThreads;  // 16-byte loads per thread and block
  extern __shared__ __attribute__((aligned(16))) uint32_t tab[];
  const int a = blockIdx.x, g = blockIdx.y, w = blockIdx.z, tid = threadIdx.x;
  const int b0 = (int)((int64_t)g * nblk / groups), b1 = (int)((int64_t)(g + 1) * nblk / groups);
  const uint32_t* sseg = sorted + (int64_t)w * Ns;
  const int start = a * kRankTile;
  const int n = min(kRankTile, N - start);
  uint32_t q[kCountItems];
  int32_t c[kCountItems];
#pragma unroll
  for (int j = 0; j < kCountItems; ++j) {
    q[j] = sseg[start + j * kCountThreads + tid];  // pad keys past n (their counts are not stored)
    c[j] = 0;
  }
  for (int c0 = b0; c0 < b1; c0 += chunk) {
    const int nb = min(chunk, b1 - c0);
    if (c0 != b0) __syncthreads();  // the previous chunk's searches are done
    // the chunk's blocks (whole, pads included): every load in flight before the first LDS write
    const u32x4* src = reinterpret_cast<const u32x4*>(sseg + (int64_t)c0 * kRankTile);
    u32x4* dst = reinterpret_cast<u32x4*>(tab);
    u32x4 v[kCountChunk * kVec];
#pragma unroll
    for (int x = 0; x < kCountChunk * kVec; ++x)
      if (x < nb * kVec) v[x] = src[x * kCountThreads + tid];
#pragma unroll
    for (int x = 0; x < kCountChunk * kVec; ++x)
      if (x < nb * kVec) dst[x * kCountThreads + tid] = v[x];
    __syncthreads();
    for (int bb = 0; bb < nb; ++bb) {
      const int b = c0 + bb;
      if (b == a) continue;
      // keys of an earlier block count when equal: compare against q + 1
      // (valid keys are at most 0x7F800000, so no wrap; a pad key wraps to 0
      // and counts nothing, which is never stored)
      const uint32_t inc = b < a ? 1u : 0u;
      const uint32_t base = (uint32_t)(bb * kRankTile * 4);  // byte offset of block bb in tab
      const char* lds = reinterpret_cast<const char*>(tab);
      const uint32_t top = *reinterpret_cast<const uint32_t*>(lds + base + 4 * (kRankTile - 1));
      uint32_t kq[kCountItems], off[kCountItems];
#pragma unroll
      for (int j = 0; j < kCountItems; ++j) {
        kq[j] = q[j] + inc;
        off[j] = base;
      }
#pragma unroll
      for (int step = kRankTile / 2; step > 0; step >>= 1)
#pragma unroll
        for (int j = 0; j < kCountItems; ++j) {
          const uint32_t e = *reinterpret_cast<const uint32_t*>(lds + off[j] + 4 * (step - 1));
          off[j] += e < kq[j] ? 4u * step : 0u;
        }
      // the search alone stops at kRankTile - 1
#pragma unroll
      for (int j = 0; j < kCountItems; ++j)
        c[j] += top < kq[j] ? kRankTile : (int)((off[j] & (kRankTile * 4 - 1)) >> 2);  // base: a multiple of 8 KB
    }
  }
  int32_t* out = part + ((int64_t)w * kRankParts + 1 + g) * N + start;
  const uint32_t* sidx = sorted_idx + (int64_t)w * Ns + start;
#pragma unroll
  for (int j = 0; j < kCountItems; ++j) {
    const int r = j * kCountThreads + tid;
    if (r < n) out[sidx[r]] = c[j];
  }
}

// Bits of select digit p of a 64-bit key: 11 bits from the top for passes
// 0-4, the low 9 bits for pass 5.
__device__ inline int sel_shift(int p) { return p < kSelPasses - 1 ? 64 - kSelBits * (p + 1) : 0; }

// Adds an LDS histogram of kSelBins counters into the global one (zeros skipped).
__device__ inline void flush_hist(const uint32_t* cnt, uint32_t* dst) {
  for (int d = threadIdx.x; d < kSelBins; d += kThreads)
    if (cnt[d]) atomicAdd(&dst[d], cnt[d]);
}

// Also the first select pass: the histogram of the top digit of s_hat, and
// the state before it (nothing fixed, keep_count to find).
__global__ __launch_bounds__(kThreads) void fuse_kernel(RankIn ranks, const float* scur, unsigned long long* shat,
                                                        double* shat_out, int N, int n_win, double lambda,
                                                        double sqrt12, uint32_t* sel_hist, SelState* states,
                                                        long long keep, const int32_t* flag) {
#pragma clang fp contract(off)
  if (*flag) return;
  __shared__ uint32_t cnt[kSelBins];
  for (int d = threadIdx.x; d < kSelBins; d += kThreads) cnt[d] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) states[0] = SelState{0ull, 0ull, keep, keep == 0, 0};
  __syncthreads();
  const int i = blockIdx.x * kThreads + threadIdx.x;
  const bool valid = i < N;
  unsigned long long bits = 0;
  if (valid) {
    const double denom = (double)(N - 1);
    double r[kMaxWindow];
    double acc = 0.0;
#pragma unroll
    for (int w = 0; w < kMaxWindow; ++w) {
      if (w < n_win) {
        int32_t rk;
        if (ranks.part[w]) {
          // every slice load in flight together: slices past n_part read slice 0 and add nothing
          int32_t c[kRankParts];
#pragma unroll
          for (int q = 0; q < kRankParts; ++q) c[q] = ranks.part[w][(int64_t)(q < ranks.n_part ? q : 0) * N + i];
          rk = 0;
#pragma unroll
          for (int q = 0; q < kRankParts; ++q) rk += q < ranks.n_part ? c[q] : 0;
          ranks.dst[w][i] = rk;
        } else {
          rk = ranks.w[w][i];
        }
        r[w] = N > 1 ? (double)rk / denom : 0.0;
        acc = acc + r[w];
      }
    }
    const double mu = acc / (double)n_win;
    double acc2 = 0.0;
#pragma unroll
    for (int w = 0; w < kMaxWindow; ++w) {
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
    if (shat_out) shat_out[i] = sh;
  }
  hist_add(cnt, (uint32_t)(bits >> sel_shift(0)), valid);
  __syncthreads();
  flush_hist(cnt, sel_hist);
}

// One select step: from the state before pass p and that pass's digit
// histogram, fix digit p (the largest digit whose suffix count reaches k_rem)
// and reduce k_rem by the count of larger digits.  Thread t owns digits
// 8t .. 8t+7; a suffix scan over the threads (within each wave, then across
// the four waves) finds the owner, which walks its digits downward; the
// result is broadcast through LDS.
__device__ SelState select_advance(SelState st, const uint32_t* hist, int p) {
  constexpr int kPer = kSelBins / kThreads;  // 8
  __shared__ uint32_t cnt[kSelBins];
  __shared__ long long wtot[kThreads / 64];
  __shared__ SelState out;
  if (st.done) return st;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int d = tid; d < kSelBins; d += kThreads) cnt[d] = hist[d];
  if (tid == 0) out = st;
  __syncthreads();
  long long own = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) own += cnt[kPer * tid + j];
  long long suf = own;  // inclusive suffix sum over the lanes >= lane of this wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long t = __shfl_down(suf, off, 64);
    if (lane + off < 64) suf += t;
  }
  if (lane == 0) wtot[wave] = suf;
  __syncthreads();
  for (int q = wave + 1; q < kThreads / 64; ++q) suf += wtot[q];
  const long long above = suf - own;
  if (above < st.k_rem && suf >= st.k_rem) {
    long long cum = above;
    for (int j = kPer - 1; j >= 0; --j) {
      const long long c = cnt[kPer * tid + j];
      if (cum + c >= st.k_rem) {
        const int shift = sel_shift(p);
        const int width = (p > 0 ? sel_shift(p - 1) : 64) - shift;
        out.prefix = st.prefix | ((unsigned long long)(kPer * tid + j) << shift);
        out.mask = st.mask | (((1ull << width) - 1ull) << shift);
        out.k_rem = st.k_rem - cum;
        out.done = out.k_rem == c || p == kSelPasses - 1;
        out.match = (int32_t)c;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  const SelState r = out;
  __syncthreads();
  return r;
}

constexpr int kFinishCap = 4096;  // keys the finishing workgroup holds in LDS

// Pass p histograms digit p of the keys that match the digits fixed so far
// (launched for p = 1 and 2).  The state before pass p is advanced once from
// the previous pass's state (stored by its workgroup 0) and histogram;
// workgroup 0 stores it in turn.  Pass 2 also appends the matching keys to
// `list` when at most kFinishCap of them match (the count of the digit pass 1
// fixed), for the finishing workgroup.
__global__ __launch_bounds__(kThreads) void select_pass_kernel(const unsigned long long* keys, int N,
                                                               uint32_t* sel_hist, SelState* states, int p,
                                                               unsigned long long* list, int32_t* list_cnt,
                                                               const int32_t* flag) {
  if (*flag) return;
  __shared__ uint32_t cnt[kSelBins];
  const SelState st = select_advance(states[p - 1], sel_hist + (p - 1) * kSelBins, p - 1);
  if (blockIdx.x == 0 && threadIdx.x == 0) states[p] = st;
  if (st.done) return;
  const bool listing = p == 2 && st.match <= kFinishCap;
  for (int d = threadIdx.x; d < kSelBins; d += kThreads) cnt[d] = 0;
  __syncthreads();
  const int shift = sel_shift(p);
  const unsigned long long dmask = (1ull << (sel_shift(p - 1) - shift)) - 1ull;
  for (int j = 0; j < kItems; ++j) {
    const int i = blockIdx.x * kSelTile + j * kThreads + threadIdx.x;
    const unsigned long long k = i < N ? keys[i] : 0ull;
    const bool match = i < N && (k & st.mask) == st.prefix;
    hist_add(cnt, (uint32_t)((k >> shift) & dmask), match);
    if (listing) {
      const unsigned long long bm = __ballot(match);
      if (bm) {
        int32_t base = 0;
        if ((threadIdx.x & 63) == 0) base = atomicAdd(list_cnt, (int32_t)__popcll(bm));
        base = __shfl(base, 0, 64);
        const int32_t at = base + (int32_t)__popcll(bm & ((1ull << (threadIdx.x & 63)) - 1ull));
        if (match && at < kFinishCap) list[at] = k;
      }
    }
  }
  __syncthreads();
  flush_hist(cnt, sel_hist + p * kSelBins);
}

// The passes after pass 2, in one workgroup: from pass 2's state and
// histogram, the final state.  When pass 2 listed the keys still matching
// (few: the first 22 bits of s_hat fix most of the order), the remaining
// passes read that list from LDS; otherwise every remaining pass scans all
// the keys.  keep == 0: the state before pass 0 is final (nothing is kept).
__global__ __launch_bounds__(kThreads) void select_finish_kernel(const unsigned long long* keys, int N,
                                                                 const uint32_t* sel_hist, SelState* states,
                                                                 const unsigned long long* glist,
                                                                 const int32_t* list_cnt, long long keep,
                                                                 const int32_t* flag) {
  if (*flag) return;
  __shared__ uint32_t hist[kSelBins];
  __shared__ unsigned long long list[kFinishCap];
  const int tid = threadIdx.x;
  if (keep == 0) {
    if (tid == 0) states[kSelPasses] = states[0];
    return;
  }
  const SelState s2 = states[2];
  const bool listed = !s2.done && s2.match <= kFinishCap;
  const int32_t n_list = listed ? min(*list_cnt, kFinishCap) : 0;
  for (int i = tid; i < n_list; i += kThreads) list[i] = glist[i];
  SelState st = select_advance(s2, sel_hist + 2 * kSelBins, 2);
  for (int p = 3; p < kSelPasses && !st.done; ++p) {
    for (int d = tid; d < kSelBins; d += kThreads) hist[d] = 0;
    __syncthreads();
    const int shift = sel_shift(p);
    const unsigned long long dmask = (1ull << (sel_shift(p - 1) - shift)) - 1ull;
    const int n = listed ? n_list : N;
    for (int i = tid; i < n; i += kThreads) {
      const unsigned long long k = listed ? list[i] : keys[i];
      if ((k & st.mask) == st.prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
    }
    __syncthreads();
    st = select_advance(st, hist, p);
  }
  if (tid == 0) states[kSelPasses] = st;
}

struct MarkArgs {
  const DevEntry* entries;
  const unsigned long long* shat;
  const uint32_t* sel_hist;
  long long keep;
  int32_t* n_gt;
  int32_t* n_eq;
  SelState* states;  // [0..5] states before each pass, [6] the final threshold
  const int32_t* flag;
};

__global__ __launch_bounds__(kThreads) void mark_kernel(MarkArgs a) {
  if (*a.flag) return;
  __shared__ int32_t sg, se;
  // threshold = the keep_count-th largest key; keep 0 keeps nothing
  const SelState st = a.states[kSelPasses];
  if (threadIdx.x == 0) { sg = 0; se = 0; }
  __syncthreads();
  const DevEntry en = a.entries[blockIdx.x];
  const int j = blockIdx.y * kThreads + threadIdx.x;
  int gt = 0, eq = 0;
  if (j < en.len) {
    const unsigned long long k = a.shat[en.tok_start + j] & st.mask;
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
  unsigned long long* host_slots;
  uint32_t slot_seq;
};

// The page's word in the host slots, if the caller asked for them.
__device__ inline void publish_slot(const CompactArgs& a, int e, uint32_t v) {
  if (a.host_slots) a.host_slots[e] = ((unsigned long long)a.slot_seq << 32) | v;
}

// Per page: which slots are kept (ties at the threshold in index order, from
// the plan step's tie rank base), the kept token ids in slot order, and the
// moves of the compaction.  With n = new length, kept slots below n stay; the
// dropped slots below n (the holes, ascending) take the kept slots at or past
// n (ascending).  Sources and destinations are disjoint, so the moves can run
// in any order.
__global__ __launch_bounds__(kThreads) void index_kernel(CompactArgs a) {
  if (const int32_t f = *a.flag) {
    if (threadIdx.x == 0) publish_slot(a, blockIdx.x, kSlotError | (uint32_t)f);
    return;
  }
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
  // thread t takes the per consecutive slots from b = t * per; its keys are
  // read once, into bit masks (bit q: slot b + q; per <= 32)
  const int per = (len + kThreads - 1) / kThreads;
  const int b = tid * per, cnt = max(0, min(per, len - b));
  const unsigned long long* sh = a.shat + en.tok_start;
  uint32_t gtm = 0, eqm = 0;
  for (int q = 0; q < cnt; ++q) {
    const unsigned long long k = sh[b + q] & st.mask;
    gtm |= (uint32_t)(k > st.prefix) << q;
    eqm |= (uint32_t)(k == st.prefix) << q;
  }
  const int32_t n_eq = __popc(eqm);
  const int32_t eq_start = eq_tot + block_excl_scan<kThreads>(n_eq, scan, nullptr);
  // keys equal to the threshold are kept in index order while fewer than
  // k_rem precede them: this thread keeps its first n_take
  const long long take = k_rem - eq_start;
  const int n_take = take <= 0 ? 0 : (take >= n_eq ? n_eq : (int)take);
  uint32_t keepm = gtm, rest = eqm;
  for (int i = 0; i < n_take; ++i) {
    const uint32_t low = rest & (0u - rest);
    keepm |= low;
    rest ^= low;
  }
  const uint32_t validm = cnt >= 32 ? 0xffffffffu : (1u << cnt) - 1u;
  const int below = max(0, min(cnt, nl - b));  // slots of this thread below nl
  const uint32_t holem = ~keepm & validm & (below >= 32 ? 0xffffffffu : (1u << below) - 1u);
  int32_t kept_total = 0, holes = 0;
  int32_t pos = block_excl_scan<kThreads>(__popc(keepm), scan, &kept_total);
  int32_t hpos = block_excl_scan<kThreads>(__popc(holem), scan, &holes);
  if (kept_total != nl) {  // cannot happen when the plan and this pass agree; never move on a mismatch
    if (tid == 0) {
      atomicOr(a.flag_rw, kClcesErrCount);
      a.n_moves[e] = 0;
      publish_slot(a, e, kSlotError | (uint32_t)kClcesErrCount);
    }
    return;
  }
  uint16_t* dst = a.move_dst + (int64_t)e * a.g.ts;
  for (int q = 0; q < cnt; ++q) {
    if ((keepm >> q) & 1u)
      kept[pos++] = (uint16_t)(b + q);
    else if ((holem >> q) & 1u)
      dst[hpos++] = (uint16_t)(b + q);
  }
  __syncthreads();
  // fillers: the kept slots at or past nl are the last `holes` entries of the kept list
  uint16_t* src = a.move_src + (int64_t)e * a.g.ts;
  for (int k = tid; k < holes; k += kThreads) src[k] = kept[nl - holes + k];
  if (a.keep_ids_out) {
    const int32_t* ids = reinterpret_cast<const int32_t*>(a.pool + (int64_t)en.phys * a.g.page_bytes + a.g.id_off);
    for (int i = tid; i < nl; i += kThreads) a.keep_ids_out[keep_base + i] = ids[kept[i]];
  }
  if (tid == 0) {
    a.n_moves[e] = holes;
    publish_slot(a, e, (uint32_t)nl);
  }
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
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t wn = (size_t)w_max * (size_t)n_max;
  z.keys = take(wn * 4);
  z.keys_b = take(wn * 4);
  z.vals_a = take(wn * 4);
  z.vals_b = take(wn * 4);
  z.blk_cnt = take((size_t)w_max * ((n_max + kRankTile - 1) / kRankTile) * 256 * 4);
  const size_t wb = (size_t)w_max * (size_t)((n_max + kRankTile - 1) / kRankTile * kRankTile);  // whole blocks
  z.sorted = take(wb * 4);
  z.sorted_idx = take(wb * 4);
  z.part = take(wn * kRankParts * 4);
  z.scur = take((size_t)n_max * 4);
  z.shat = take((size_t)n_max * 8);
  z.sel_hist = take((size_t)kSelPasses * kSelBins * 4);
  z.sel_state = take((kSelPasses + 1) * sizeof(SelState));
  z.list = take(kFinishCap * sizeof(unsigned long long));
  z.list_cnt = take(4);
  z.entries = take((size_t)p_max * sizeof(DevEntry));
  z.counts = take((size_t)p_max * 2 * 4);
  z.move_src = take((size_t)p_max * ts_max * 2);
  z.move_dst = take((size_t)p_max * ts_max * 2);
  z.n_moves = take((size_t)p_max * 4);
  z.flag = take(((size_t)p_max + 1) * 4);  // the error flag, then the new page lengths [p_max]
  z.total = off;
  return z;
}

hipError_t launch_rank_sort_count(const uint32_t* keys, uint32_t* sorted, uint32_t* sorted_idx, int32_t* part, int N,
                                int segments, const int32_t* flag, int* n_part, hipStream_t s) {
  const int nblk = (N + kRankTile - 1) / kRankTile;
  const int64_t Ns = (int64_t)nblk * kRankTile;
  const int groups = nblk > 1 ? std::min(nblk, (int)kRankGroups) : 0;
  rank_sort_kernel<<<dim3((unsigned)nblk, (unsigned)segments), dim3(kRankThreads), 0, s>>>(keys, sorted, sorted_idx,
                                                                                          part, N, Ns, flag);
  if (groups > 0) {
    const int chunk = std::min((nblk + groups - 1) / groups, kCountChunk);  // the largest group, or a chunk of it
    rank_count_kernel<<<dim3((unsigned)nblk, (unsigned)groups, (unsigned)segments), dim3(kCountThreads),
                        (size_t)chunk * kRankTile * sizeof(uint32_t), s>>>(sorted, sorted_idx, part, N, Ns, nblk,
                                                                           groups, chunk, flag);
  }
  *n_part = 1 + groups;
  return hipGetLastError();
}

hipError_t launch_rank_radix(uint32_t* keys_a, uint32_t* keys_b, uint32_t* vals_a, uint32_t* vals_b, uint32_t* blk_cnt,
                             int32_t* const* dst, int N, int segments, const int32_t* flag, hipStream_t s) {
  const int nblk = (N + kRankTile - 1) / kRankTile;
  RankOut out{};
  for (int w = 0; w < segments; ++w) out.seg[w] = dst[w];
  uint32_t* kin = keys_a;
  uint32_t* kout = keys_b;
  uint32_t* vin = nullptr;
  uint32_t* vout = vals_b;
  const dim3 grid((unsigned)nblk, (unsigned)segments);
  for (int pass = 0; pass < 4; ++pass) {
    rank_hist_kernel<<<grid, dim3(kHistThreads), 0, s>>>(kin, blk_cnt, N, nblk, pass, flag);
    rank_scatter_kernel<<<grid, dim3(kRankThreads), 0, s>>>(kin, vin, kout, vout, blk_cnt, out, N, nblk, pass, flag);
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
  auto* keys = reinterpret_cast<uint32_t*>(ws + z.keys);
  auto* part = reinterpret_cast<int32_t*>(ws + z.part);
  auto* scur = reinterpret_cast<float*>(ws + z.scur);
  auto* shat = reinterpret_cast<unsigned long long*>(ws + z.shat);
  auto* sel_hist = reinterpret_cast<uint32_t*>(ws + z.sel_hist);
  auto* sel_state = reinterpret_cast<SelState*>(ws + z.sel_state);
  auto* counts = reinterpret_cast<int32_t*>(ws + z.counts);
  auto* flag = reinterpret_cast<int32_t*>(ws + z.flag);
  const int P = a.n_entries, N = a.n_tokens, W = a.n_window;
  if (P > z.p_max || (int64_t)N > z.n_max || W > z.w_max || W > kMaxWindow || a.n_rank > W ||
      a.geom.ts > kMaxPageTokensScored)
    return hipErrorInvalidValue;

  {
    TableChunk c;
    c.first = 0;
    c.count = std::min(P, kUploadChunk);
    for (int i = 0; i < c.count; ++i) c.e[i] = a.entries_host[i];
    const int n_hist = kSelPasses * kSelBins;
    const int64_t nz = std::max(n_hist, 2 * P);
    prep_kernel<<<dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, s>>>(
        entries, c, sel_hist, n_hist, counts, 2 * P, reinterpret_cast<int32_t*>(ws + z.list_cnt), flag);
  }
  hipError_t e = P > kUploadChunk ? launch_table_upload(entries + kUploadChunk, a.entries_host + kUploadChunk,
                                                        P - kUploadChunk, s)
                                  : hipGetLastError();
  if (e != hipSuccess) return e;

  // raw scores: the layers to rank (window slots with rank_out set), then the current layer
  GatherArgs g{};
  g.entries = entries;
  g.pool = a.pool;
  g.page_bytes = a.geom.page_bytes;
  g.id_off = a.geom.id_off;
  g.table = a.score_table;
  g.rows = a.score_rows;
  g.cols = a.score_cols;
  g.col_cur = a.first_layer + W - 1;
  g.N = N;
  g.keys = keys;
  g.scur = scur;
  g.flag = flag;
  // Window slot w ranked in this step is segment nseg of the gathered keys.
  // Block sort + counts: its count slices sum to its rank in fuse, which
  // stores it at rank_dst[w]; radix passes: the rank goes to rank_dst[w].
  const int64_t nblk_rank = (N + kRankTile - 1) / kRankTile;
  const bool radix = a.rank_radix || (int64_t)a.n_rank * nblk_rank * nblk_rank > kSortCountMax;
  RankIn ri{};
  int32_t* dst[kMaxWindow] = {};
  int nseg = 0;
  for (int w = 0; w < W; ++w) {
    if (a.rank_new[w]) {
      g.seg_col[nseg] = a.first_layer + w;
      dst[nseg] = a.rank_dst[w];
      if (!radix) {
        ri.part[w] = part + (int64_t)nseg * kRankParts * N;
        ri.dst[w] = a.rank_dst[w];
      } else {
        ri.w[w] = a.rank_dst[w];
      }
      ++nseg;
    } else {
      ri.w[w] = a.rank_dst[w];
    }
  }
  g.n_seg = nseg;
  gather_kernel<<<dim3((unsigned)P, (unsigned)((a.geom.ts + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(g);
  if (nseg > 0) {
    e = radix ? launch_rank_radix(keys, reinterpret_cast<uint32_t*>(ws + z.keys_b),
                                  reinterpret_cast<uint32_t*>(ws + z.vals_a), reinterpret_cast<uint32_t*>(ws + z.vals_b),
                                  reinterpret_cast<uint32_t*>(ws + z.blk_cnt), dst, N, nseg, flag, s)
              : launch_rank_sort_count(keys, reinterpret_cast<uint32_t*>(ws + z.sorted),
                                       reinterpret_cast<uint32_t*>(ws + z.sorted_idx), part, N, nseg, flag,
                                       &ri.n_part, s);
    if (e != hipSuccess) return e;
  }
  fuse_kernel<<<dim3((unsigned)((N + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(
      ri, scur, shat, a.s_hat_out, N, W, a.lambda, std::sqrt(12.0), sel_hist, sel_state, a.keep, flag);
  const int nblk = (N + kSelTile - 1) / kSelTile;
  unsigned long long* list = reinterpret_cast<unsigned long long*>(ws + z.list);
  int32_t* list_cnt = reinterpret_cast<int32_t*>(ws + z.list_cnt);
  if (a.keep > 0)
    for (int p = 1; p <= 2; ++p)
      select_pass_kernel<<<dim3((unsigned)nblk), dim3(kThreads), 0, s>>>(shat, N, sel_hist, sel_state, p, list,
                                                                        list_cnt, flag);
  select_finish_kernel<<<dim3(1), dim3(kThreads), 0, s>>>(shat, N, sel_hist, sel_state, list, list_cnt, a.keep,
                                                          flag);
  MarkArgs m{entries, shat, sel_hist, a.keep, counts, counts + P, sel_state, flag};
  mark_kernel<<<dim3((unsigned)P, (unsigned)((a.geom.ts + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(m);
  CompactArgs ca{entries,
                 reinterpret_cast<uint16_t*>(ws + z.move_src),
                 reinterpret_cast<uint16_t*>(ws + z.move_dst),
                 reinterpret_cast<int32_t*>(ws + z.n_moves),
                 shat, sel_state + kSelPasses, counts, counts + P, flag + 1, P, a.pool, a.geom, a.keep_ids_out, flag,
                 flag, a.host_slots, a.slot_seq};
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

}  // namespace kvs
