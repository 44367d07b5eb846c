// Diversity-scored per-head pruning, gfx950.
//
// InfiniteVGGT explainer ("InfiniteVGGT: Visual Geometry Grounded Transformer
// for Endless Streams"): "Building Blocks" (diversity = negative cosine
// similarity of a key to the mean key; a per-layer, per-head top-K keeps the
// most diverse tokens), "Cosine Similarity" (keys are L2-normalised and
// compared by direction) and the step-by-step recipe, steps 2-6 (the
// candidates are the mutable cache, never the anchor; the reference is the
// mean of the normalised candidate keys).  With S the sum of the normalised
// candidate keys of a head, the mean is S / N, so the score of key k is
// -(k . S) / (|k| |S|); a zero key, or a zero S, scores 0.
//
// One call covers several layers at once: every kernel runs over all of them
// (the last grid dimension is the layer's slot), so a 24-layer step is about
// a dozen launches.  The sum and score kernels run one workgroup per (page,
// head, slot); 8 threads share a key row (8 of its 64 dims each) and the row
// sums are completed with butterfly shuffles, so every lane of a row holds the
// same bits.  The mark and compact kernels run one workgroup per (page,
// slot), one wave per head at a time.  Every sum has a fixed order, so results are bit-reproducible
// from run to run.
//   tables  per (head, slot): candidate pages, the head's rows in each and
//           the prefixes, from the layer's shared table and the per-page
//           head lengths;
//   sum     float64 sum over a page's rows of k / |k|;
//   mean    per (head, slot): the pages' sums added in a fixed order = S,
//           and |S|;
//   score   float64 score per row (the value that is ranked and reported),
//           stored as a 64-bit key that orders the scores descending, split
//           in a high and a low 32-bit plane; float64 score sums per block;
//   total   per slot, the block sums added in a fixed order;
//   select  one workgroup per (head, slot), up to 8 radix passes of 8 bits
//           in one launch (most significant first; the first four read only
//           the high plane) find the K-th smallest key t and how many keys
//           equal to t are kept: the first ones in candidate order, as a
//           stable sort would keep them.  Once every key matching the digits
//           fixed so far is kept, the remaining passes are skipped and t
//           compares under the mask of the fixed bits; once few keys match,
//           they are copied to LDS and the later passes read only those;
//   mark    per (page, head, slot): keys below t and equal to t;
//   compact per (page, head, slot): the page's new length n follows from the
//           counts; kept = key < t, or key == t within the tie quota; the
//           dropped slots below n take the kept slots at or past n (both
//           ascending), moving the head's K and V rows, and n goes to the
//           per-page head-length array that the attention tables use.
// Each layer's keys stay in its own part of the key store, so a prune that
// follows a scoring of the same, unchanged layer starts at the select.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "blockscan.h"
#include "clces.h"
#include "diversity.h"
#include "rowmove.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;
constexpr int kTPR = 8;                        // threads per key row
constexpr int kRowsPerPass = kThreads / kTPR;  // 32

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Select state of one head: the key bits fixed so far (prefix, under mask)
// and how many of the keys matching them are still to be kept.  done: no
// further pass is needed (every matching key is kept, or none is to be kept,
// or all 64 bits are fixed).
struct DSel {
  uint64_t prefix;
  uint64_t mask;
  long long k_rem;
  int32_t done;
  int32_t pad;
};
constexpr int kDivSelPasses = 8;

struct DivK {
  const DivLayer* layers;  // [n]
  const DevEntry* bases;   // [n][p_max]
  DevEntry* tabs;          // [n][H][p_max + 1]; entry P: tok_start = the head's candidate count
  int32_t n, p_max, H;
  char* pool;
  int64_t page_bytes, k_off, v_off;
  int32_t ts;
  double* partial;  // [n][H][p_max][64]
  double* mean;     // [n][H][65]: S, then |S|
  double* spart;    // [n][H][p_max]
  double* totals;   // [n]
  uint32_t* keys;   // the key store: per layer and head a high plane [N], then a low plane [N]
  double* scores;   // optional [H][score_stride] of slot 0
  int64_t score_stride;
  DSel* dstate;     // [n][H] final select states
  uint32_t* hist0;  // [layer][H][256] counts of each key's top byte (the first select digit), per pool layer
  int32_t* lt_cnt;  // [n][H][p_max] keys below the threshold per page
  int32_t* eq_cnt;  // [n][H][p_max] keys equal to the threshold per page
  int32_t* new_len; // [n][items_p][H]
  int32_t items_p;  // pages per slot in the launch grids (the call's largest P)
  int32_t* hcount;    // [n][H] candidates per head (the tables kernel's totals)
  int32_t* kept;      // [n][H] kept candidates per head (the compaction's new lengths added up)
  int32_t* hlen;    // [phys][H]
  int32_t* flags;   // [n] per slot, [n] the call's
};

__device__ inline const DevEntry& tab(const DivK& a, int slot, int h, int p) {
  return a.tabs[((int64_t)slot * a.H + h) * (a.p_max + 1) + p];
}
// High plane of head h's keys; the low plane follows at + L.N.
__device__ inline uint32_t* head_keys(const DivK& a, const DivLayer& L, int h) {
  return a.keys + L.keys_off + (int64_t)h * 2 * L.N;
}

// One workgroup per (head, slot): head h's table from the layer's shared one
// (an entry with tile_start != 0 takes its length from hlen[phys * H + h]).
__global__ __launch_bounds__(kThreads) void div_tables_kernel(DivK a) {
  __shared__ int32_t scan[kThreads];
  const int h = blockIdx.x, slot = blockIdx.y, tid = threadIdx.x;
  const int n = a.layers[slot].P;
  const DevEntry* base = a.bases + (int64_t)slot * a.p_max;
  DevEntry* t = a.tabs + ((int64_t)slot * a.H + h) * (a.p_max + 1);
  const int per = (n + kThreads - 1) / kThreads;
  const int b = min(tid * per, n), e = min(b + per, n);
  auto len_of = [&](const DevEntry& be) { return be.tile_start ? a.hlen[(int64_t)be.phys * a.H + h] : be.len; };
  int32_t toks = 0;
  for (int i = b; i < e; ++i) toks += len_of(base[i]);
  int32_t total = 0;
  int32_t k0 = block_excl_scan<kThreads>(toks, scan, &total);
  for (int i = b; i < e; ++i) {
    const DevEntry be = base[i];
    const int32_t len = len_of(be);
    t[i] = DevEntry{be.phys, len, 0, k0};
    k0 += len;
  }
  if (tid == 0) {
    t[n] = DevEntry{0, 0, 0, total};
    a.hcount[(int64_t)slot * a.H + h] = total;
  }
  // the score kernel of this call counts the first select digit afresh
  if (a.layers[slot].rescore) a.hist0[((int64_t)a.layers[slot].layer * a.H + h) * 256 + tid] = 0u;
}

// The call's staging block (parameters and candidate pages, written by the
// host into pinned memory) copied into the workspace, 16 bytes per thread,
// and the error flags cleared.  A kernel reads the pinned block directly:
// no separate copy operation has to start before the first kernel.
__global__ void div_stage_kernel(const int4* src, int4* dst, int n16, int32_t* flags, int n_flags) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) dst[i] = src[i];
  if (i < n_flags) flags[i] = 0;
}

// The 8 elements c*8 .. c*8+7 of one row as loaded (one 16-byte vector for
// bf16, two for fp32), then widened to float64.
template <typename T>
struct RowPart {
  V16 v[sizeof(T) / 2];
};

template <typename T>
__device__ inline RowPart<T> load_part(const char* row, int c) {
  RowPart<T> r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i)
    r.v[i] = *reinterpret_cast<const V16*>(row + c * 8 * (int)sizeof(T) + 16 * i);
  return r;
}

__device__ inline void widen(const RowPart<__bf16>& r, double (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = (uint32_t)r.v[0][i];
    x[2 * i] = (double)__uint_as_float(w << 16);
    x[2 * i + 1] = (double)__uint_as_float(w & 0xffff0000u);
  }
}

__device__ inline void widen(const RowPart<float>& r, double (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = (double)__int_as_float(r.v[0][i]);
    x[4 + i] = (double)__int_as_float(r.v[1][i]);
  }
}

// Rows of a page that one thread loads before it uses the first: enough
// bytes in flight per wave to cover the memory latency.
constexpr int kUnroll = 4;

// The parts of rows j0 + u * kRowsPerPass + r (u < kUnroll) this thread reads;
// rows past len read as zero.
template <typename T>
__device__ inline void load_rows(const char* rows, int j0, int r, int c, int len, RowPart<T> (&raw)[kUnroll]) {
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int j = j0 + u * kRowsPerPass + r;
    if (j < len) {
      raw[u] = load_part<T>(rows + (int64_t)j * kHeadDim * sizeof(T), c);
    } else {
#pragma unroll
      for (int i = 0; i < (int)(sizeof(T) / 2); ++i) raw[u].v[i] = V16{0, 0, 0, 0};
    }
  }
}

// A double moved across lanes by one DPP pattern (both halves).
template <int CTRL>
__device__ inline double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}

// Sum over the 8 lanes of a row (an aligned group of 8 lanes): quad
// permutes swap lanes 1 apart and 2 apart, then the half-row mirror pairs
// each lane of one quad with a lane of the other.  Every lane ends with the
// same bits (each level adds the same two operands, in either order).
__device__ inline double row_sum(double v) {
  v += dpp_f64<0xb1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4e>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  return v;
}

template <typename T>
__device__ inline const char* key_rows(const DivK& a, const DevEntry& en, int h) {
  return a.pool + (int64_t)en.phys * a.page_bytes + a.k_off + (int64_t)h * a.ts * kHeadDim * (int64_t)sizeof(T);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void div_sum_kernel(DivK a) {
#pragma clang fp contract(off)
  __shared__ double red[kRowsPerPass][kHeadDim + 1];
  const int p = blockIdx.x, h = blockIdx.y, slot = blockIdx.z, tid = threadIdx.x;
  const DivLayer L = a.layers[slot];
  if (!L.rescore || p >= L.P) return;
  const int r = tid / kTPR, c = tid % kTPR;
  const DevEntry en = tab(a, slot, h, p);
  const char* rows = key_rows<T>(a, en, h);
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  for (int j0 = 0; j0 < en.len; j0 += kRowsPerPass * kUnroll) {
    RowPart<T> raw[kUnroll];
    load_rows<T>(rows, j0, r, c, en.len, raw);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      double x[8];
      widen(raw[u], x);
      double s2 = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) s2 = s2 + x[i] * x[i];
      s2 = row_sum(s2);
      if (s2 > 0.0) {
        const double inv = 1.0 / sqrt(s2);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = acc[i] + x[i] * inv;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[r][c * 8 + i] = acc[i];
  __syncthreads();
  if (tid < kHeadDim) {
    double s = 0.0;
    for (int q = 0; q < kRowsPerPass; ++q) s = s + red[q][tid];
    a.partial[(((int64_t)slot * a.H + h) * a.p_max + p) * kHeadDim + tid] = s;
  }
}

// One workgroup per (head, slot): 16 groups of 64 threads (one per dim) each
// add every 16th page's sum in table order, then the groups' sums are added
// in group order.
constexpr int kMeanThreads = 1024;
constexpr int kMeanGroups = kMeanThreads / kHeadDim;

__global__ __launch_bounds__(kMeanThreads) void div_mean_kernel(DivK a) {
#pragma clang fp contract(off)
  __shared__ double red[kMeanGroups][kHeadDim];
  const int h = blockIdx.x, slot = blockIdx.y, tid = threadIdx.x;
  const DivLayer L = a.layers[slot];
  if (!L.rescore) return;
  const int g = tid / kHeadDim, d = tid % kHeadDim;
  const double* part = a.partial + ((int64_t)slot * a.H + h) * a.p_max * kHeadDim;
  double s = 0.0;
  for (int p = g; p < L.P; p += kMeanGroups) s = s + part[(int64_t)p * kHeadDim + d];
  red[g][d] = s;
  __syncthreads();
  if (tid < kHeadDim) {
    s = 0.0;
    for (int q = 0; q < kMeanGroups; ++q) s = s + red[q][tid];
    double* m = a.mean + ((int64_t)slot * a.H + h) * (kHeadDim + 1);
    m[tid] = s;
    double sq = s * s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) sq += __shfl_xor(sq, off, 64);
    if (tid == 0) m[kHeadDim] = sqrt(sq);
  }
}

// Add one to bin d of the LDS histogram for every lane with valid set.  The
// wave's lanes are grouped by digit for up to two distinct digits (one LDS
// atomic per group); lanes with further digits add one each.  The first
// select digits take only a few values (sign and exponent bits), and
// same-address atomics from many lanes, which the LDS serialises, are avoided.
__device__ inline void hist_add2(uint32_t* cnt, uint32_t d, bool valid) {
  unsigned long long left = __ballot(valid);
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    if (!left) return;
    const int first = __ffsll((long long)left) - 1;
    const uint32_t lead = (uint32_t)__builtin_amdgcn_readlane((int)d, first);
    const unsigned long long same = __ballot(valid && d == lead) & left;
    if (lane == first) atomicAdd(&cnt[lead], (uint32_t)__popcll(same));
    left &= ~same;
  }
  if ((left >> lane) & 1ull) atomicAdd(&cnt[d], 1u);
}

// Rank key of a float64 score: ascending keys = descending scores (-0 as +0).
__device__ inline uint64_t desc_key(double f) {
  if (f == 0.0) f = 0.0;
  const uint64_t b = (uint64_t)__double_as_longlong(f);
  const uint64_t asc = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
  return ~asc;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void div_score_kernel(DivK a) {
#pragma clang fp contract(off)
  __shared__ double red[kThreads];
  __shared__ uint32_t h0[256];
  const int p = blockIdx.x, h = blockIdx.y, slot = blockIdx.z, tid = threadIdx.x;
  const DivLayer L = a.layers[slot];
  if (!L.rescore || p >= L.P) return;
  const int r = tid / kTPR, c = tid % kTPR;
  h0[tid] = 0u;
  __syncthreads();
  const DevEntry en = tab(a, slot, h, p);
  const char* rows = key_rows<T>(a, en, h);
  const double* m = a.mean + ((int64_t)slot * a.H + h) * (kHeadDim + 1);
  double sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = m[c * 8 + i];
  const double sn = m[kHeadDim];
  uint32_t* kk = head_keys(a, L, h);
  double ssum = 0.0;
  bool bad = false;
  static_assert(kUnroll <= kTPR, "one lane of a row group per unrolled row");
  for (int j0 = 0; j0 < en.len; j0 += kRowsPerPass * kUnroll) {
    RowPart<T> raw[kUnroll];
    load_rows<T>(rows, j0, r, c, en.len, raw);
    double s2u[kUnroll], dotu[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      double x[8];
      widen(raw[u], x);
      double s2 = 0.0, dot = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s2 = s2 + x[i] * x[i];
        dot = dot + x[i] * sv[i];
      }
      // every lane of the row group holds the same sums afterwards
      s2u[u] = row_sum(s2);
      dotu[u] = row_sum(dot);
    }
    // lane u of each row group finishes unrolled row u: the square root and
    // the division run once for kUnroll rows
    uint32_t digit0 = 0u;
    bool counted = false;
    if (c < kUnroll) {
      double s2 = s2u[0], dot = dotu[0];
#pragma unroll
      for (int u = 1; u < kUnroll; ++u)
        if (c == u) {
          s2 = s2u[u];
          dot = dotu[u];
        }
      const int j = j0 + c * kRowsPerPass + r;
      if (j < en.len) {
        const double sc = (s2 > 0.0 && sn > 0.0) ? -(dot / (sqrt(s2) * sn)) : 0.0;
        bad = bad || !(s2 <= 1.0e300) || !(sc == sc);  // a NaN or infinite key
        const int64_t idx = en.tok_start + j;
        const uint64_t key = desc_key(sc);
        kk[idx] = (uint32_t)(key >> 32);
        kk[L.N + idx] = (uint32_t)key;
        digit0 = (uint32_t)(key >> 56);
        counted = true;
        if (a.scores && slot == 0) a.scores[(int64_t)h * a.score_stride + idx] = sc;
        ssum = ssum + sc;
      }
    }
    hist_add2(h0, digit0, counted);
  }
  if (__ballot(bad) != 0ull && (tid & 63) == 0) {
    atomicOr(&a.flags[slot], kDivErrNan);
    atomicOr(&a.flags[a.n], kDivErrNan);
  }
  red[tid] = ssum;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] = red[tid] + red[tid + off];
    __syncthreads();
  }
  if (tid == 0) a.spart[((int64_t)slot * a.H + h) * a.p_max + p] = red[0];
  if (h0[tid]) atomicAdd(&a.hist0[((int64_t)L.layer * a.H + h) * 256 + tid], h0[tid]);
}

// One workgroup per slot: the block sums of every head and page, in a fixed order.
__global__ __launch_bounds__(kThreads) void div_total_kernel(DivK a) {
#pragma clang fp contract(off)
  __shared__ double red[kThreads];
  const int slot = blockIdx.x, tid = threadIdx.x;
  const DivLayer L = a.layers[slot];
  if (!L.rescore) return;
  double s = 0.0;
  for (int h = 0; h < a.H; ++h) {
    const double* sp = a.spart + ((int64_t)slot * a.H + h) * a.p_max;
    for (int p = tid; p < L.P; p += kThreads) s = s + sp[p];
  }
  red[tid] = s;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] = red[tid] + red[tid + off];
    __syncthreads();
  }
  if (tid == 0) a.totals[slot] = red[0];
}

// The select runs one workgroup of kSelThreads per (head, slot) through all
// its passes in one launch: the histogram of each pass and the choice of its
// digit stay in LDS.  Pass p histograms digit p (bits 56 - 8p .. 63 - 8p) of
// the keys that match the digits fixed so far, then fixes it: the smallest
// digit whose prefix count (over digits in ascending order) reaches k_rem;
// k_rem drops by the count of the smaller digits.  When every key matching
// the new prefix is to be kept, no later pass can change the outcome (done).
// Once at most kSelListCap keys match the prefix, the pass that reads them
// also copies them (64-bit) into LDS, and the later passes read that list.
constexpr int kSelThreads = 512;
constexpr int kSelBatch = 16;      // keys per thread in flight
constexpr int kSelListCap = 7168;  // keys listed in LDS (56 KB)

__global__ __launch_bounds__(kSelThreads) void div_select_kernel(DivK a) {
  extern __shared__ uint64_t sel_list[];  // [kSelListCap]
  __shared__ uint32_t cnt[256];
  __shared__ DSel s_st;
  __shared__ long long s_c;
  __shared__ int32_t s_n;
  const int h = blockIdx.x, slot = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  if (a.flags[a.n]) return;
  const DivLayer L = a.layers[slot];
  const int64_t nh = a.hcount[(int64_t)slot * a.H + h];
  const long long k0 = (long long)min<int64_t>(L.keep, nh);
  DSel st{0ull, 0ull, k0, k0 == 0 || k0 == nh, 0};
  const uint32_t* kh = head_keys(a, L, h);
  const uint32_t* kl = kh + L.N;
  bool listed = false;      // the keys matching the prefix are in sel_list (s_n of them)
  long long c_match = nh;   // keys matching the prefix
  for (int p = 0; p < kDivSelPasses && !st.done; ++p) {
    const bool listing = p > 0 && !listed && c_match <= kSelListCap;
    const bool need_lo = p >= 4 || listing;
    const int shift = 56 - 8 * p;
    const uint32_t pre_hi = (uint32_t)(st.prefix >> 32), mask_hi = (uint32_t)(st.mask >> 32);
    // pass 0 takes the counts the score kernel made of the same keys
    if (tid < 256) cnt[tid] = p == 0 ? a.hist0[((int64_t)L.layer * a.H + h) * 256 + tid] : 0u;
    if (tid == 0 && listing) s_n = 0;
    __syncthreads();
    if (p == 0) {
    } else if (listed) {
      const int n_list = min(s_n, kSelListCap);
      for (int i = tid; i < n_list; i += kSelThreads) {
        const uint64_t key = sel_list[i];
        if ((key & st.mask) == st.prefix) atomicAdd(&cnt[(uint32_t)(key >> shift) & 255u], 1u);
      }
    } else {
      for (int64_t b = 0; b < nh; b += (int64_t)kSelThreads * kSelBatch) {
        const int64_t i0 = b + tid;
        uint32_t hi[kSelBatch], lo[kSelBatch];
        bool match[kSelBatch];
        // every load of the batch is issued before any key is counted
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) hi[j] = i0 + j * kSelThreads < nh ? kh[i0 + j * kSelThreads] : 0u;
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
          match[j] = i0 + j * kSelThreads < nh && (hi[j] & mask_hi) == pre_hi;
          lo[j] = 0u;
        }
        // low words of the matching keys; the other lanes all read the
        // plane's first word (one shared line), so the loads need no branch
        if (need_lo) {
#pragma unroll
          for (int j = 0; j < kSelBatch; ++j) lo[j] = kl[match[j] ? i0 + j * kSelThreads : 0];
        }
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
          const uint64_t key = ((uint64_t)hi[j] << 32) | lo[j];
          const bool m = match[j] && (key & st.mask) == st.prefix;
          // the first digit (sign and exponent bits) takes few values: group
          // the lanes; later digits are spread: one atomic per lane
          if (p == 0)
            hist_add2(cnt, (uint32_t)(key >> shift) & 255u, m);
          else if (m)
            atomicAdd(&cnt[(uint32_t)(key >> shift) & 255u], 1u);
          if (listing) {
            const unsigned long long bm = __ballot(m);
            if (bm) {
              int32_t base = 0;
              if (lane == 0) base = atomicAdd(&s_n, (int32_t)__popcll(bm));
              base = __builtin_amdgcn_readfirstlane(base);
              const int32_t at = base + (int32_t)__popcll(bm & ((1ull << lane) - 1ull));
              if (m && at < kSelListCap) sel_list[at] = key;
            }
          }
        }
      }
    }
    __syncthreads();
    // fix digit p (wave 0: 4 digits per lane, inclusive prefix over lanes)
    if (tid < 64) {
      if (tid == 0) {
        s_st = st;
        s_st.done = 1;  // kept if no digit reaches k_rem (inconsistent counts)
        s_c = 0;
      }
      uint32_t c4[4];
      long long own = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c4[j] = cnt[4 * tid + j];
        own += c4[j];
      }
      long long pre = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const long long t = __shfl_up(pre, off, 64);
        if (tid >= off) pre += t;
      }
      const long long below = pre - own;
      if (below < st.k_rem && pre >= st.k_rem) {
        long long cum = below;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum + c4[j] >= st.k_rem) {
            DSel out = st;
            out.prefix = st.prefix | ((uint64_t)(4 * tid + j) << shift);
            out.mask = st.mask | (0xffull << shift);
            out.k_rem = st.k_rem - cum;
            out.done = out.k_rem == (long long)c4[j] || p == kDivSelPasses - 1;
            s_st = out;
            s_c = c4[j];
            break;
          }
          cum += c4[j];
        }
      }
    }
    __syncthreads();
    st = s_st;
    c_match = s_c;
    listed = listed || listing;
    __syncthreads();  // s_st and s_c are rewritten by the next pass
  }
  if (tid == 0) a.dstate[(int64_t)slot * a.H + h] = st;
}

// Candidate i's key under the final state's mask against the threshold
// prefix: -1 below, 0 equal, 1 above.  hi is the key's high word; the low
// word is read only when the high words match under the mask.
__device__ inline int key_cmp(uint32_t hi, const uint32_t* kl, int64_t i, const DSel& st) {
  const uint32_t h = hi & (uint32_t)(st.mask >> 32), ph = (uint32_t)(st.prefix >> 32);
  if (h != ph) return h < ph ? -1 : 1;
  const uint32_t ml = (uint32_t)st.mask;
  if (!ml) return 0;
  const uint32_t l = kl[i] & ml, pl = (uint32_t)st.prefix;
  return l == pl ? 0 : (l < pl ? -1 : 1);
}

// The mark and compact kernels run one workgroup per (page, slot) of up to
// 4 waves (more waves per workgroup measured slower: fewer workgroups in
// flight per CU); wave w takes heads w, w + waves, ..., and loads 512 of a
// head's keys (8 per lane) before it compares them.
constexpr int kMaxItemWaves = 4;
constexpr int kBatch = 8;

// Per (page, head, slot): the keys below the threshold t and equal to it.
__global__ __launch_bounds__(64 * kMaxItemWaves) void div_mark_kernel(DivK a) {
  if (a.flags[a.n]) return;
  const int p = blockIdx.x, slot = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int waves = blockDim.x >> 6;
  const DivLayer L = a.layers[slot];
  if (p >= L.P) return;
  for (int h = wave; h < a.H; h += waves) {
    const DSel st = a.dstate[(int64_t)slot * a.H + h];
    const DevEntry en = tab(a, slot, h, p);
    const uint32_t* kh = head_keys(a, L, h) + en.tok_start;
    const uint32_t* kl = kh + L.N;
    int32_t lt = 0, eq = 0;
    for (int j0 = 0; j0 < en.len; j0 += 64 * kBatch) {
      uint32_t hi[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = j0 + 64 * u + lane;
        hi[u] = j < en.len ? kh[j] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = j0 + 64 * u + lane;
        const int c = j < en.len ? key_cmp(hi[u], kl, j, st) : 1;
        lt += __popcll(__ballot(c < 0));
        eq += __popcll(__ballot(c == 0));
      }
    }
    if (lane == 0) {
      const int64_t at = ((int64_t)slot * a.H + h) * a.p_max + p;
      a.lt_cnt[at] = lt;
      a.eq_cnt[at] = eq;
    }
  }
}

// Per (page, head, slot), one wave: the new length n (keys below t, plus the
// page's share of the tie quota), then, walking the page in 64-slot chunks
// with ballots, the dropped slots below n and the kept slots at or past n in
// ascending order (lists in the wave's part of LDS, max_moves entries each),
// and the row moves between them.  The lists are written and read by the
// same wave, whose LDS accesses complete in order.
template <typename T>
__global__ __launch_bounds__(64 * kMaxItemWaves) void div_compact_kernel(DivK a, int max_moves) {
  if (a.flags[a.n]) return;
  extern __shared__ uint16_t move_lists[];  // [wave][2][max_moves]: holes, then fills
  const int p = blockIdx.x, slot = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int waves = blockDim.x >> 6;
  const DivLayer L = a.layers[slot];
  if (p >= L.P) return;
  uint16_t* holes = move_lists + (size_t)wave * 2 * max_moves;
  uint16_t* fills = holes + max_moves;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int h = wave; h < a.H; h += waves) {
    const DevEntry en = tab(a, slot, h, p);
    const int len = en.len;
    const DSel st = a.dstate[(int64_t)slot * a.H + h];
    const int64_t cnt_at = ((int64_t)slot * a.H + h) * a.p_max;
    const int32_t eq = a.eq_cnt[cnt_at + p];
    // keys equal to t in the earlier pages: only a page holding such a key
    // needs them (its share of the tie quota)
    long long eq_before = 0;
    if (eq > 0) {
      int32_t e = 0;
      for (int q = lane; q < p; q += 64) e += a.eq_cnt[cnt_at + q];
      for (int off = 32; off > 0; off >>= 1) e += __shfl_xor(e, off, 64);
      eq_before = e;
    }
    const long long quota = st.k_rem - eq_before;
    const int32_t n = a.lt_cnt[cnt_at + p] + (int32_t)(quota < 0 ? 0 : (quota > eq ? eq : quota));
    if (lane == 0) {
      a.new_len[((int64_t)slot * a.items_p + p) * a.H + h] = n;
      a.hlen[(int64_t)en.phys * a.H + h] = n;
    }
    if (n == len) continue;  // nothing dropped in this page and head
    const uint32_t* kh = head_keys(a, L, h) + en.tok_start;
    const uint32_t* kl = kh + L.N;
    long long eq_run = eq_before;
    int32_t h_run = 0, f_run = 0;
    for (int j0 = 0; j0 < len; j0 += 64 * kBatch) {
      uint32_t hi[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = j0 + 64 * u + lane;
        hi[u] = j < len ? kh[j] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int j = j0 + 64 * u + lane;
        const bool valid = j < len;
        const int c = valid ? key_cmp(hi[u], kl, j, st) : 1;
        const unsigned long long be = __ballot(c == 0);
        const bool keep = c < 0 || (c == 0 && eq_run + __popcll(be & below) < st.k_rem);
        const bool hole = valid && !keep && j < n;
        const bool fill = keep && j >= n;
        const unsigned long long bh = __ballot(hole), bf = __ballot(fill);
        const int32_t hp = h_run + __popcll(bh & below), fp = f_run + __popcll(bf & below);
        // a consistent plan has at most len / 2 moves; the counts are checked below
        if (hole && hp < max_moves) holes[hp] = (uint16_t)j;
        if (fill && fp < max_moves) fills[fp] = (uint16_t)j;
        eq_run += __popcll(be);
        h_run += __popcll(bh);
        f_run += __popcll(bf);
      }
    }
    // cannot happen when the counts and the walk agree; never move on a mismatch
    if (h_run != f_run || h_run > max_moves) {
      if (lane == 0) atomicOr(&a.flags[slot], kClcesErrCount);
      continue;
    }
    __builtin_amdgcn_wave_barrier();
    constexpr int VPR = kHeadDim * sizeof(T) / 16;
    char* page = a.pool + (int64_t)en.phys * a.page_bytes;
    move_rows<T, 64>(reinterpret_cast<V16*>(page + a.k_off) + (int64_t)h * a.ts * VPR, fills, holes, h_run, lane);
    move_rows<T, 64>(reinterpret_cast<V16*>(page + a.v_off) + (int64_t)h * a.ts * VPR, fills, holes, h_run, lane);
    __builtin_amdgcn_wave_barrier();  // the next head's lists are written after these reads
  }
}

// One workgroup per (head, slot): the head's kept total, its new lengths
// added over the pages (checked against min(keep, candidates) on the host).
__global__ __launch_bounds__(kThreads) void div_kept_kernel(DivK a) {
  __shared__ int32_t red[kThreads];
  const int h = blockIdx.x, slot = blockIdx.y, tid = threadIdx.x;
  const int P = a.layers[slot].P;
  int32_t k = 0;
  for (int p = tid; p < P; p += kThreads) k += a.new_len[((int64_t)slot * a.items_p + p) * a.H + h];
  red[tid] = k;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  if (tid == 0) a.kept[(int64_t)slot * a.H + h] = red[0];
}

DivK make_k(const DivCall& c) {
  const DivSizes& z = c.sizes;
  DivK k{};
  k.layers = reinterpret_cast<const DivLayer*>(c.ws + z.params);
  k.bases = reinterpret_cast<const DevEntry*>(c.ws + z.bases);
  k.tabs = reinterpret_cast<DevEntry*>(c.ws + z.tabs);
  k.n = c.n;
  k.p_max = z.p_max;
  k.items_p = c.max_P;
  k.H = c.geom.heads;
  k.pool = c.pool;
  k.page_bytes = c.geom.page_bytes;
  k.k_off = c.geom.k_off;
  k.v_off = c.geom.v_off;
  k.ts = c.geom.ts;
  k.partial = reinterpret_cast<double*>(c.ws + z.partial);
  k.mean = reinterpret_cast<double*>(c.ws + z.mean);
  k.spart = reinterpret_cast<double*>(c.ws + z.spart);
  k.totals = reinterpret_cast<double*>(c.ws + z.totals);
  k.keys = c.keys_dev;
  k.scores = c.scores_out;
  k.score_stride = c.score_stride;
  k.dstate = reinterpret_cast<DSel*>(c.ws + z.dstate);
  k.hist0 = reinterpret_cast<uint32_t*>(c.ws + z.hist0);
  k.lt_cnt = reinterpret_cast<int32_t*>(c.ws + z.lt_cnt);
  k.eq_cnt = reinterpret_cast<int32_t*>(c.ws + z.eq_cnt);
  k.new_len = reinterpret_cast<int32_t*>(c.ws + z.new_len);
  k.hcount = reinterpret_cast<int32_t*>(c.ws + z.hcount);
  k.kept = reinterpret_cast<int32_t*>(c.ws + z.kept);
  k.hlen = c.hlen_dev;
  k.flags = reinterpret_cast<int32_t*>(c.ws + z.flags);
  return k;
}

}  // namespace

DivSizes div_sizes(int64_t n_max, int32_t p_max, int32_t heads, int32_t layers) {
  DivSizes z{};
  z.n_max = n_max;
  z.p_max = p_max;
  z.h_max = heads;
  z.layers = layers;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t L = (size_t)layers, H = (size_t)heads, P = (size_t)p_max;
  z.params = take(L * sizeof(DivLayer));
  z.bases = take(L * P * sizeof(DevEntry));
  z.tabs = take(L * H * (P + 1) * sizeof(DevEntry));
  z.partial = take(L * H * P * kHeadDim * 8);
  z.mean = take(L * H * (kHeadDim + 1) * 8);
  z.spart = take(L * H * P * 8);
  z.dstate = take(L * H * sizeof(DSel));
  z.hist0 = take(L * H * 256 * 4);
  z.lt_cnt = take(L * H * P * 4);
  z.eq_cnt = take(L * H * P * 4);
  // the outputs the host reads back, adjacent (no alignment padding between
  // them): a scoring reads totals, flags and head counts in one copy; a prune
  // flags, head counts, kept totals and new lengths in one copy
  z.totals = take(L * 8);
  z.flags = z.totals + L * 8;
  z.hcount = z.flags + (L + 1) * 4;
  z.kept = z.hcount + L * H * 4;
  z.new_len = z.kept + L * H * 4;
  off = align256(z.new_len + L * P * H * 4);
  z.total = off;
  return z;
}

size_t div_staging_bytes(const DivSizes& z, int n) {
  return (z.bases - z.params) + (size_t)n * z.p_max * sizeof(DevEntry);
}

hipError_t enqueue_diversity(const DivCall& c, hipStream_t s) {
  const DivSizes& z = c.sizes;
  if (c.n < 1 || c.n > z.layers || c.max_P < 1 || c.max_P > z.p_max || c.geom.heads > z.h_max || c.max_N < 1 ||
      c.max_N > z.n_max || c.geom.ts > kMaxPageTokensScored)
    return hipErrorInvalidValue;
  const DivK k = make_k(c);
  const int H = c.geom.heads;
  const int n16 = (int)((div_staging_bytes(z, c.n) + 15) / 16);
  div_stage_kernel<<<dim3((unsigned)((std::max(n16, c.n + 1) + 255) / 256)), dim3(256), 0, s>>>(
      reinterpret_cast<const int4*>(c.staging), reinterpret_cast<int4*>(c.ws + z.params), n16, k.flags, c.n + 1);
  div_tables_kernel<<<dim3((unsigned)H, (unsigned)c.n), dim3(kThreads), 0, s>>>(k);
  const dim3 pages((unsigned)c.max_P, (unsigned)H, (unsigned)c.n);
  if (c.any_rescore) {
    if (c.geom.esize == 2)
      div_sum_kernel<__bf16><<<pages, dim3(kThreads), 0, s>>>(k);
    else
      div_sum_kernel<float><<<pages, dim3(kThreads), 0, s>>>(k);
    div_mean_kernel<<<dim3((unsigned)H, (unsigned)c.n), dim3(kMeanThreads), 0, s>>>(k);
    if (c.geom.esize == 2)
      div_score_kernel<__bf16><<<pages, dim3(kThreads), 0, s>>>(k);
    else
      div_score_kernel<float><<<pages, dim3(kThreads), 0, s>>>(k);
    div_total_kernel<<<dim3((unsigned)c.n), dim3(kThreads), 0, s>>>(k);
  }
  if (c.prune) {
    div_select_kernel<<<dim3((unsigned)H, (unsigned)c.n), dim3(kSelThreads), kSelListCap * sizeof(uint64_t), s>>>(k);
    const dim3 page_grid((unsigned)c.max_P, (unsigned)c.n);
    div_mark_kernel<<<page_grid, dim3(64 * std::min(H, kMaxItemWaves)), 0, s>>>(k);
    // one wave per head (up to 4), as many as 64 KB of move lists allow
    const int max_moves = std::max(1, c.geom.ts / 2);
    const size_t per_wave = 2 * (size_t)max_moves * sizeof(uint16_t);
    const int waves = std::max(1, std::min({H, kMaxItemWaves, (int)((64 << 10) / per_wave)}));
    if (c.geom.esize == 2)
      div_compact_kernel<__bf16><<<page_grid, dim3(64 * waves), waves * per_wave, s>>>(k, max_moves);
    else
      div_compact_kernel<float><<<page_grid, dim3(64 * waves), waves * per_wave, s>>>(k, max_moves);
    div_kept_kernel<<<dim3((unsigned)H, (unsigned)c.n), dim3(kThreads), 0, s>>>(k);
  }
  return hipGetLastError();
}

}  // namespace kvs
