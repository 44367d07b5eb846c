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
// a dozen launches.  Page-level kernels run one workgroup per (page, head,
// slot); 8 threads share a key row (8 of its 64 dims each) and the row sums
// are completed with butterfly shuffles, so every lane of a row holds the
// same bits.  Every sum has a fixed order, so results are bit-reproducible
// from run to run.
//   tables  per (head, slot): candidate pages, the head's rows in each and
//           the prefixes, from the layer's shared table and the per-page
//           head lengths;
//   sum     float64 sum over a page's rows of k / |k|;
//   mean    per (head, slot): the pages' sums added in a fixed order = S,
//           and |S|;
//   score   float64 score per row, rounded to float32 (the value that is
//           ranked and reported) and stored as a 32-bit key that orders the
//           scores descending; float64 score sums per block;
//   total   per slot, the block sums added in a fixed order;
//   select  per (head, slot), 4 radix passes of 8 bits (most significant
//           first) find the K-th smallest key t and how many keys equal to t
//           are kept: the first ones in candidate order, as a stable sort
//           would keep them (a histogram pass over the keys, then one
//           workgroup per (head, slot) fixes the digit);
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
constexpr int kMaxMoves = kMaxPageTokensScored / 2;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Select state of one head: the key prefix fixed so far and how many of the
// keys matching it are still to be kept.
struct DSel {
  uint32_t prefix;
  int32_t pad;
  long long k_rem;
};

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
  uint32_t* keys;   // the key store
  float* scores;    // optional [H][score_stride] of slot 0
  int64_t score_stride;
  uint32_t* dhist;  // [n][4][H][256] select histograms
  DSel* dstate;     // [n][5][H] states before each pass, [4] final
  int32_t* lt_cnt;  // [n][H][p_max] keys below the threshold per page
  int32_t* eq_cnt;  // [n][H][p_max] keys equal to the threshold per page
  int32_t* new_len; // [n][p_max][H]
  int32_t* hlen;    // [phys][H]
  int32_t* flags;   // [n] per slot, [n] the call's
};

__device__ inline const DevEntry& tab(const DivK& a, int slot, int h, int p) {
  return a.tabs[((int64_t)slot * a.H + h) * (a.p_max + 1) + p];
}
__device__ inline int64_t head_count(const DivK& a, int slot, int h) {
  return tab(a, slot, h, a.layers[slot].P).tok_start;
}
__device__ inline uint32_t* head_keys(const DivK& a, const DivLayer& L, int h) {
  return a.keys + L.keys_off + (int64_t)h * L.N;
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
  if (tid == 0) t[n] = DevEntry{0, 0, 0, total};
}

__global__ void div_zero_kernel(int32_t* p0, int n0, int32_t* p1, int n1) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n0) p0[i] = 0;
  if (i < n1) p1[i] = 0;
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

// Rank key of a score: ascending keys = descending scores (-0 as +0).
__device__ inline uint32_t desc_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t b = __float_as_uint(f);
  const uint32_t asc = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ~asc;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void div_score_kernel(DivK a) {
#pragma clang fp contract(off)
  __shared__ double red[kThreads];
  const int p = blockIdx.x, h = blockIdx.y, slot = blockIdx.z, tid = threadIdx.x;
  const DivLayer L = a.layers[slot];
  if (!L.rescore || p >= L.P) return;
  const int r = tid / kTPR, c = tid % kTPR;
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
        const float f = (float)sc;
        const int64_t idx = en.tok_start + j;
        kk[idx] = desc_key(f);
        if (a.scores && slot == 0) a.scores[(int64_t)h * a.score_stride + idx] = f;
        ssum = ssum + sc;
      }
    }
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

constexpr int kSelItems = 8;
constexpr int kSelTile = kThreads * kSelItems;

// Fix digit p: the smallest digit whose prefix count (over digits in
// ascending order) reaches k_rem; k_rem drops by the count of smaller digits.
// Wave 0 scans its 64 lanes (4 digits each); the result goes through LDS.
// Every thread of the (256-thread) workgroup calls it.
__device__ DSel select_advance(DSel st, const uint32_t* hist, int p) {
  __shared__ uint32_t cnt[256];
  __shared__ DSel out;
  const int tid = threadIdx.x;
  cnt[tid] = hist[tid];
  if (tid == 0) out = st;
  __syncthreads();
  if (tid < 64 && st.k_rem > 0) {
    long long own = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) own += cnt[4 * tid + j];
    long long pre = own;  // inclusive prefix over lanes <= tid
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long t = __shfl_up(pre, off, 64);
      if (tid >= off) pre += t;
    }
    const long long below = pre - own;
    if (below < st.k_rem && pre >= st.k_rem) {
      long long cum = below;
      for (int j = 0; j < 4; ++j) {
        const long long c = cnt[4 * tid + j];
        if (cum + c >= st.k_rem) {
          out.prefix = st.prefix | ((uint32_t)(4 * tid + j) << (24 - 8 * p));
          out.k_rem = st.k_rem - cum;
          break;
        }
        cum += c;
      }
    }
  }
  __syncthreads();
  const DSel r = out;
  __syncthreads();
  return r;
}

__device__ inline uint32_t* sel_hist(const DivK& a, int slot, int p, int h) {
  return a.dhist + (((int64_t)slot * 4 + p) * a.H + h) * 256;
}
__device__ inline DSel* sel_state(const DivK& a, int slot, int p, int h) {
  return a.dstate + ((int64_t)slot * 5 + p) * a.H + h;
}

// One workgroup per (head, slot): the state before pass p (p = 0: nothing
// fixed, min(keep, candidates) to keep; p = 1..4: pass p-1's state advanced
// by its histogram; state 4 is the final one).
__global__ __launch_bounds__(kThreads) void div_advance_kernel(DivK a, int p) {
  if (a.flags[a.n]) return;
  const int h = blockIdx.x, slot = blockIdx.y;
  const DSel st = p == 0 ? DSel{0u, 0, (long long)min<int64_t>(a.layers[slot].keep, head_count(a, slot, h))}
                         : select_advance(*sel_state(a, slot, p - 1, h), sel_hist(a, slot, p - 1, h), p - 1);
  if (threadIdx.x == 0) *sel_state(a, slot, p, h) = st;
}

// Pass p: histogram of digit p over head h's keys that match the digits
// fixed so far.
__global__ __launch_bounds__(kThreads) void div_select_kernel(DivK a, int p) {
  if (a.flags[a.n]) return;
  __shared__ uint32_t cnt[256];
  const int h = blockIdx.y, slot = blockIdx.z, tid = threadIdx.x;
  const int64_t nh = head_count(a, slot, h);
  if ((int64_t)blockIdx.x * kSelTile >= nh) return;  // past the head's keys
  const DSel st = *sel_state(a, slot, p, h);
  if (st.k_rem == 0) return;
  cnt[tid] = 0;
  __syncthreads();
  const int shift = 24 - 8 * p;
  const uint32_t hi = p == 0 ? 0u : (~0u << (32 - 8 * p));
  const uint32_t* kk = head_keys(a, a.layers[slot], h);
#pragma unroll
  for (int j = 0; j < kSelItems; ++j) {
    const int64_t i = (int64_t)blockIdx.x * kSelTile + j * kThreads + tid;
    const uint32_t key = i < nh ? kk[i] : 0u;
    hist_add(cnt, (key >> shift) & 255u, i < nh && (key & hi) == st.prefix);
  }
  __syncthreads();
  if (cnt[tid]) atomicAdd(&sel_hist(a, slot, p, h)[tid], cnt[tid]);
}

// Per (page, head, slot): the keys below the threshold t and equal to it.
__global__ __launch_bounds__(kThreads) void div_mark_kernel(DivK a) {
  if (a.flags[a.n]) return;
  __shared__ int32_t s_lt, s_eq;
  const int p = blockIdx.x, h = blockIdx.y, slot = blockIdx.z, tid = threadIdx.x;
  const DivLayer L = a.layers[slot];
  if (p >= L.P) return;
  const uint32_t t = sel_state(a, slot, 4, h)->prefix;
  if (tid == 0) {
    s_lt = 0;
    s_eq = 0;
  }
  __syncthreads();
  const DevEntry en = tab(a, slot, h, p);
  const uint32_t* kk = head_keys(a, L, h) + en.tok_start;
  int32_t lt = 0, eq = 0;
  for (int j = tid; j < en.len; j += kThreads) {
    const uint32_t key = kk[j];
    lt += key < t;
    eq += key == t;
  }
  for (int off = 32; off > 0; off >>= 1) {
    lt += __shfl_xor(lt, off, 64);
    eq += __shfl_xor(eq, off, 64);
  }
  if ((tid & 63) == 0) {
    if (lt) atomicAdd(&s_lt, lt);
    if (eq) atomicAdd(&s_eq, eq);
  }
  __syncthreads();
  if (tid == 0) {
    const int64_t at = ((int64_t)slot * a.H + h) * a.p_max + p;
    a.lt_cnt[at] = s_lt;
    a.eq_cnt[at] = s_eq;
  }
}

// Per (page, head, slot): the new length n (keys below t, plus the page's
// share of the tie quota), then, walking the page in chunks of 256 slots with
// wave ballots, the dropped slots below n and the kept slots at or past n in
// ascending order, and the row moves between them.
template <typename T>
__global__ __launch_bounds__(kThreads) void div_compact_kernel(DivK a) {
  if (a.flags[a.n]) return;
  constexpr int kWaves = kThreads / 64;
  __shared__ int32_t s_eqb;
  __shared__ int32_t wsum[3][kWaves];
  __shared__ uint16_t holes[kMaxMoves], fills[kMaxMoves];
  const int p = blockIdx.x, h = blockIdx.y, slot = blockIdx.z, tid = threadIdx.x;
  const DivLayer L = a.layers[slot];
  if (p >= L.P) return;
  const int wave = tid >> 6, lane = tid & 63;
  const DevEntry en = tab(a, slot, h, p);
  const int len = en.len;
  const DSel st = *sel_state(a, slot, 4, h);
  const int64_t cnt_at = ((int64_t)slot * a.H + h) * a.p_max;
  const int32_t eq = a.eq_cnt[cnt_at + p];
  // keys equal to t in the earlier pages: only a page holding such a key
  // needs them (its share of the tie quota), and such pages are rare
  if (tid == 0) s_eqb = 0;
  __syncthreads();
  if (eq > 0) {
    int32_t e = 0;
    for (int i = tid; i < p; i += kThreads) e += a.eq_cnt[cnt_at + i];
    if (e) atomicAdd(&s_eqb, e);
    __syncthreads();
  }
  const long long eq_before = s_eqb;
  const long long quota = st.k_rem - eq_before;
  const int32_t n = a.lt_cnt[cnt_at + p] + (int32_t)(quota < 0 ? 0 : (quota > eq ? eq : quota));
  if (tid == 0) {
    a.new_len[((int64_t)slot * a.p_max + p) * a.H + h] = n;
    a.hlen[(int64_t)en.phys * a.H + h] = n;
  }
  if (n == len) return;  // nothing dropped in this page and head
  const uint32_t* kk = head_keys(a, L, h) + en.tok_start;
  const unsigned long long below = (1ull << lane) - 1ull;
  long long eq_run = eq_before;
  int32_t h_run = 0, f_run = 0;
  for (int c0 = 0; c0 < len; c0 += kThreads) {
    const int j = c0 + tid;
    const bool valid = j < len;
    const uint32_t key = valid ? kk[j] : 0xffffffffu;
    const bool is_eq = valid && key == st.prefix;
    const unsigned long long be = __ballot(is_eq);
    if (lane == 0) wsum[0][wave] = __popcll(be);
    __syncthreads();
    long long eq_rank = eq_run + __popcll(be & below);
    int32_t chunk_eq = 0;
    for (int w = 0; w < kWaves; ++w) {
      eq_rank += w < wave ? wsum[0][w] : 0;
      chunk_eq += wsum[0][w];
    }
    const bool keep = valid && (key < st.prefix || (is_eq && eq_rank < st.k_rem));
    const bool hole = valid && !keep && j < n;
    const bool fill = keep && j >= n;
    const unsigned long long bh = __ballot(hole), bf = __ballot(fill);
    if (lane == 0) {
      wsum[1][wave] = __popcll(bh);
      wsum[2][wave] = __popcll(bf);
    }
    __syncthreads();
    int32_t hp = h_run + __popcll(bh & below), fp = f_run + __popcll(bf & below);
    int32_t chunk_h = 0, chunk_f = 0;
    for (int w = 0; w < kWaves; ++w) {
      hp += w < wave ? wsum[1][w] : 0;
      fp += w < wave ? wsum[2][w] : 0;
      chunk_h += wsum[1][w];
      chunk_f += wsum[2][w];
    }
    if (hole) holes[hp] = (uint16_t)j;
    if (fill) fills[fp] = (uint16_t)j;
    eq_run += chunk_eq;
    h_run += chunk_h;
    f_run += chunk_f;
    __syncthreads();  // wsum is rewritten by the next chunk; the lists are read below
  }
  if (h_run != f_run) {  // cannot happen when the counts and the walk agree; never move on a mismatch
    if (tid == 0) atomicOr(&a.flags[slot], kClcesErrCount);
    return;
  }
  constexpr int VPR = kHeadDim * sizeof(T) / 16;
  char* page = a.pool + (int64_t)en.phys * a.page_bytes;
  move_rows<T, kThreads>(reinterpret_cast<V16*>(page + a.k_off) + (int64_t)h * a.ts * VPR, fills, holes, h_run, tid);
  move_rows<T, kThreads>(reinterpret_cast<V16*>(page + a.v_off) + (int64_t)h * a.ts * VPR, fills, holes, h_run, tid);
}

DivK make_k(const DivCall& c) {
  const DivSizes& z = c.sizes;
  DivK k{};
  k.layers = reinterpret_cast<const DivLayer*>(c.ws + z.params);
  k.bases = reinterpret_cast<const DevEntry*>(c.ws + z.bases);
  k.tabs = reinterpret_cast<DevEntry*>(c.ws + z.tabs);
  k.n = c.n;
  k.p_max = z.p_max;
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
  k.dhist = reinterpret_cast<uint32_t*>(c.ws + z.dhist);
  k.dstate = reinterpret_cast<DSel*>(c.ws + z.dstate);
  k.lt_cnt = reinterpret_cast<int32_t*>(c.ws + z.lt_cnt);
  k.eq_cnt = reinterpret_cast<int32_t*>(c.ws + z.eq_cnt);
  k.new_len = reinterpret_cast<int32_t*>(c.ws + z.new_len);
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
  z.dhist = take(L * 4 * H * 256 * 4);
  z.dstate = take(L * 5 * H * sizeof(DSel));
  z.lt_cnt = take(L * H * P * 4);
  z.eq_cnt = take(L * H * P * 4);
  // the outputs the host reads back, adjacent: a scoring reads totals and
  // flags in one copy, a prune flags and new lengths in one copy
  z.totals = take(L * 8);
  z.flags = take((L + 1) * 4);
  z.new_len = take(L * P * H * 4);
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
  hipError_t e = hipMemcpyAsync(c.ws + z.params, c.staging, div_staging_bytes(z, c.n), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return e;
  const int n_hist = c.prune ? c.n * 4 * H * 256 : 0;
  div_zero_kernel<<<dim3((unsigned)((std::max(n_hist, c.n + 1) + 255) / 256)), dim3(256), 0, s>>>(
      k.flags, c.n + 1, reinterpret_cast<int32_t*>(k.dhist), n_hist);
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
    const unsigned nblk = (unsigned)((c.max_N + kSelTile - 1) / kSelTile);
    const dim3 heads((unsigned)H, (unsigned)c.n);
    for (int p = 0; p < 4; ++p) {
      div_advance_kernel<<<heads, dim3(kThreads), 0, s>>>(k, p);
      div_select_kernel<<<dim3(nblk, (unsigned)H, (unsigned)c.n), dim3(kThreads), 0, s>>>(k, p);
    }
    div_advance_kernel<<<heads, dim3(kThreads), 0, s>>>(k, 4);
    div_mark_kernel<<<pages, dim3(kThreads), 0, s>>>(k);
    if (c.geom.esize == 2)
      div_compact_kernel<__bf16><<<pages, dim3(kThreads), 0, s>>>(k);
    else
      div_compact_kernel<float><<<pages, dim3(kThreads), 0, s>>>(k);
  }
  return hipGetLastError();
}

}  // namespace kvs
