// Diversity-scored per-head pruning of one layer, gfx950.
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
// Pipeline over one layer (one launch each, all on the caller's stream, one
// final sync).  Every (page, head) pair is a workgroup; 8 threads share a key
// row (8 of its 64 dims each) and the row sums are completed with butterfly
// shuffles, so every lane of a row holds the same bits.  Every sum has a
// fixed order, so results are bit-reproducible from run to run.
//   tables  per head: candidate pages, the head's rows in each, prefixes;
//   sum     float64 sum over the page's rows of k / |k|;
//   mean    per head: the pages' sums added in table order = S, and |S|;
//           pads the head's rank keys past its candidate count;
//   score   float64 score per row, rounded to float32 (the value that is
//           ranked and reported); float64 score sums per block;
//   total   the block sums added in a fixed order (one workgroup);
//   rank    stable LSD radix rank per head of the descending-score keys, so
//           ties go to the lower candidate index;
//   compact per (page, head): kept = rank < K; with n kept in the page, the
//           dropped slots below n take the kept slots at or past n (both
//           ascending); K and V rows move, and the head's new length goes to
//           the per-page head-length array that the attention tables use.

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

struct DivK {
  const DevEntry* tabs;  // [H][P + 1]; entry P: tok_start = the head's candidate count
  int32_t P, H;
  int64_t N;  // rank segment length (the largest candidate count)
  char* pool;
  int64_t page_bytes, k_off, v_off;
  int32_t ts;
  double* partial;  // [H][P][64]
  double* mean;     // [H][64] S, then [H] |S| at mean + 64 * H
  double* spart;    // [H][P]
  double* total;    // [1]
  uint32_t* keys;   // [H][N]
  float* scores;    // optional [H][score_stride]
  int64_t score_stride;
  const int32_t* ranks;  // [H][N]
  int64_t keep;
  int32_t* new_len;  // [P][H]
  int32_t* hlen;     // [phys][H]
  int32_t* flag;
};

// The 8 elements c*8 .. c*8+7 of one row, as float64.
template <typename T>
__device__ inline void load8(const char* row, int c, double (&x)[8]);

template <>
__device__ inline void load8<__bf16>(const char* row, int c, double (&x)[8]) {
  const V16 v = *reinterpret_cast<const V16*>(row + c * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = (uint32_t)v[i];
    x[2 * i] = (double)__uint_as_float(w << 16);
    x[2 * i + 1] = (double)__uint_as_float(w & 0xffff0000u);
  }
}

template <>
__device__ inline void load8<float>(const char* row, int c, double (&x)[8]) {
  const V16 a = *reinterpret_cast<const V16*>(row + c * 32);
  const V16 b = *reinterpret_cast<const V16*>(row + c * 32 + 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = (double)__int_as_float(a[i]);
    x[4 + i] = (double)__int_as_float(b[i]);
  }
}

// Sum over the 8 lanes of a row; every lane ends with the same bits (each
// level adds the same two operands, in either order).
__device__ inline double row_sum(double v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
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
  const int p = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = tid / kTPR, c = tid % kTPR;
  const DevEntry en = a.tabs[(int64_t)h * (a.P + 1) + p];
  const char* rows = key_rows<T>(a, en, h);
  double acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0;
  for (int j0 = 0; j0 < en.len; j0 += kRowsPerPass) {
    const int j = j0 + r;
    double x[8];
    if (j < en.len) {
      load8<T>(rows + (int64_t)j * kHeadDim * sizeof(T), c, x);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.0;
    }
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
#pragma unroll
  for (int i = 0; i < 8; ++i) red[r][c * 8 + i] = acc[i];
  __syncthreads();
  if (tid < kHeadDim) {
    double s = 0.0;
    for (int q = 0; q < kRowsPerPass; ++q) s = s + red[q][tid];
    a.partial[((int64_t)h * a.P + p) * kHeadDim + tid] = s;
  }
}

// One workgroup per head.
__global__ __launch_bounds__(kThreads) void div_mean_kernel(DivK a) {
#pragma clang fp contract(off)
  const int h = blockIdx.x, tid = threadIdx.x;
  if (tid < kHeadDim) {
    double s = 0.0;
    for (int p = 0; p < a.P; ++p) s = s + a.partial[((int64_t)h * a.P + p) * kHeadDim + tid];
    a.mean[(int64_t)h * kHeadDim + tid] = s;
    double q = s * s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) q += __shfl_xor(q, off, 64);
    if (tid == 0) a.mean[(int64_t)a.H * kHeadDim + h] = sqrt(q);
  }
  const int64_t nh = a.tabs[(int64_t)h * (a.P + 1) + a.P].tok_start;
  for (int64_t i = nh + tid; i < a.N; i += kThreads) a.keys[(int64_t)h * a.N + i] = 0xffffffffu;
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
  const int p = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int r = tid / kTPR, c = tid % kTPR;
  const DevEntry en = a.tabs[(int64_t)h * (a.P + 1) + p];
  const char* rows = key_rows<T>(a, en, h);
  double sv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sv[i] = a.mean[(int64_t)h * kHeadDim + c * 8 + i];
  const double sn = a.mean[(int64_t)a.H * kHeadDim + h];
  double ssum = 0.0;
  bool bad = false;
  for (int j0 = 0; j0 < en.len; j0 += kRowsPerPass) {
    const int j = j0 + r;
    double x[8];
    if (j < en.len) {
      load8<T>(rows + (int64_t)j * kHeadDim * sizeof(T), c, x);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.0;
    }
    double s2 = 0.0, dot = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s2 = s2 + x[i] * x[i];
      dot = dot + x[i] * sv[i];
    }
    s2 = row_sum(s2);
    dot = row_sum(dot);
    if (j < en.len && c == 0) {
      const double sc = (s2 > 0.0 && sn > 0.0) ? -((dot / sqrt(s2)) / sn) : 0.0;
      bad = bad || !(s2 <= 1.0e300) || !(sc == sc);  // a NaN or infinite key
      const float f = (float)sc;
      const int64_t idx = en.tok_start + j;
      a.keys[(int64_t)h * a.N + idx] = desc_key(f);
      if (a.scores) a.scores[(int64_t)h * a.score_stride + idx] = f;
      ssum = ssum + sc;
    }
  }
  if (__ballot(bad) != 0ull && (tid & 63) == 0) atomicOr(a.flag, kDivErrNan);
  red[tid] = ssum;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] = red[tid] + red[tid + off];
    __syncthreads();
  }
  if (tid == 0) a.spart[(int64_t)h * a.P + p] = red[0];
}

__global__ __launch_bounds__(kThreads) void div_total_kernel(DivK a) {
#pragma clang fp contract(off)
  __shared__ double red[kThreads];
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)a.H * a.P;
  double s = 0.0;
  for (int64_t i = tid; i < n; i += kThreads) s = s + a.spart[i];
  red[tid] = s;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] = red[tid] + red[tid + off];
    __syncthreads();
  }
  if (tid == 0) *a.total = red[0];
}

template <typename T>
__global__ __launch_bounds__(kThreads) void div_compact_kernel(DivK a) {
  if (*a.flag) return;
  __shared__ int32_t scan[kThreads];
  __shared__ uint16_t holes[kMaxMoves], fills[kMaxMoves];
  const int p = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const DevEntry en = a.tabs[(int64_t)h * (a.P + 1) + p];
  const int len = en.len;
  const int32_t* rk = a.ranks + (int64_t)h * a.N + en.tok_start;
  const int per = (len + kThreads - 1) / kThreads;
  const int b = min(tid * per, len), end = min(b + per, len);
  int32_t nk = 0;
  for (int j = b; j < end; ++j) nk += (int64_t)rk[j] < a.keep;
  int32_t n = 0;
  block_excl_scan<kThreads>(nk, scan, &n);
  int32_t nh = 0, nf = 0;
  for (int j = b; j < end; ++j) {
    const bool kept = (int64_t)rk[j] < a.keep;
    nh += !kept && j < n;
    nf += kept && j >= n;
  }
  int32_t n_holes = 0;
  int32_t hp = block_excl_scan<kThreads>(nh, scan, &n_holes);
  int32_t fp = block_excl_scan<kThreads>(nf, scan, nullptr);
  for (int j = b; j < end; ++j) {
    const bool kept = (int64_t)rk[j] < a.keep;
    if (!kept && j < n) holes[hp++] = (uint16_t)j;
    if (kept && j >= n) fills[fp++] = (uint16_t)j;
  }
  if (tid == 0) {
    a.new_len[(int64_t)p * a.H + h] = n;
    a.hlen[(int64_t)en.phys * a.H + h] = n;
  }
  __syncthreads();
  if (n_holes == 0) return;
  constexpr int VPR = kHeadDim * sizeof(T) / 16;
  char* page = a.pool + (int64_t)en.phys * a.page_bytes;
  move_rows<T, kThreads>(reinterpret_cast<V16*>(page + a.k_off) + (int64_t)h * a.ts * VPR, fills, holes, n_holes,
                         tid);
  move_rows<T, kThreads>(reinterpret_cast<V16*>(page + a.v_off) + (int64_t)h * a.ts * VPR, fills, holes, n_holes,
                         tid);
}

DivK make_k(const DivArgs& a) {
  const DivSizes& z = a.sizes;
  DivK k{};
  k.tabs = reinterpret_cast<const DevEntry*>(a.ws + z.entries);
  k.P = a.P;
  k.H = a.geom.heads;
  k.N = a.N;
  k.pool = a.pool;
  k.page_bytes = a.geom.page_bytes;
  k.k_off = a.geom.k_off;
  k.v_off = a.geom.v_off;
  k.ts = a.geom.ts;
  k.partial = reinterpret_cast<double*>(a.ws + z.partial);
  k.mean = reinterpret_cast<double*>(a.ws + z.mean);
  k.spart = reinterpret_cast<double*>(a.ws + z.spart);
  k.total = reinterpret_cast<double*>(a.ws + z.total_sum);
  k.keys = reinterpret_cast<uint32_t*>(a.ws + z.keys_a);
  k.scores = a.scores_out;
  k.score_stride = a.score_stride;
  k.ranks = reinterpret_cast<const int32_t*>(a.ws + z.ranks);
  k.keep = a.keep;
  k.new_len = reinterpret_cast<int32_t*>(a.ws + z.new_len);
  k.hlen = a.hlen_dev;
  k.flag = reinterpret_cast<int32_t*>(a.ws + z.flag);
  return k;
}

__global__ void div_flag_clear_kernel(int32_t* flag) { *flag = 0; }

// Tables, flag, sums, mean and scores: the part both entry points share.
hipError_t enqueue_scores(const DivArgs& a, const DivK& k, hipStream_t s) {
  const DivSizes& z = a.sizes;
  const int H = a.geom.heads;
  if (a.P < 1 || a.P > z.p_max || H > z.h_max || a.N < 1 || a.N > z.n_max || a.geom.ts > kMaxPageTokensScored)
    return hipErrorInvalidValue;
  DevEntry* base = reinterpret_cast<DevEntry*>(a.ws + z.entries) + (int64_t)H * (a.P + 1);
  hipError_t e = launch_table_upload(base, a.base_host, a.P, s);
  if (e != hipSuccess) return e;
  e = launch_head_tables(const_cast<DevEntry*>(k.tabs), base, a.P, a.hlen_dev, H, s);
  if (e != hipSuccess) return e;
  div_flag_clear_kernel<<<1, 1, 0, s>>>(k.flag);
  const dim3 grid((unsigned)a.P, (unsigned)H);
  if (a.geom.esize == 2)
    div_sum_kernel<__bf16><<<grid, dim3(kThreads), 0, s>>>(k);
  else
    div_sum_kernel<float><<<grid, dim3(kThreads), 0, s>>>(k);
  div_mean_kernel<<<dim3((unsigned)H), dim3(kThreads), 0, s>>>(k);
  if (a.geom.esize == 2)
    div_score_kernel<__bf16><<<grid, dim3(kThreads), 0, s>>>(k);
  else
    div_score_kernel<float><<<grid, dim3(kThreads), 0, s>>>(k);
  div_total_kernel<<<1, dim3(kThreads), 0, s>>>(k);
  return hipGetLastError();
}

hipError_t finish(const DivArgs& a, const DivK& k, int32_t* new_len_host, double* score_sum_host,
                  int32_t* err_flag_host, hipStream_t s) {
  hipError_t e;
  if (new_len_host) {
    e = hipMemcpyAsync(new_len_host, k.new_len, sizeof(int32_t) * (size_t)a.P * a.geom.heads,
                       hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return e;
  }
  e = hipMemcpyAsync(score_sum_host, k.total, sizeof(double), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  e = hipMemcpyAsync(err_flag_host, k.flag, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

}  // namespace

DivSizes div_sizes(int64_t n_max, int32_t p_max, int32_t heads) {
  DivSizes z{};
  z.n_max = n_max;
  z.p_max = p_max;
  z.h_max = heads;
  z.nblk_max = (int32_t)((n_max + kRankTile - 1) / kRankTile);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t hn = (size_t)heads * (size_t)n_max;
  const size_t hp = (size_t)heads * (size_t)p_max;
  z.entries = take(((size_t)heads * (p_max + 1) + (size_t)p_max) * sizeof(DevEntry));
  z.partial = take(hp * kHeadDim * 8);
  z.mean = take((size_t)heads * (kHeadDim + 1) * 8);
  z.spart = take(hp * 8);
  z.total_sum = take(8);
  z.keys_a = take(hn * 4);
  z.keys_b = take(hn * 4);
  z.vals_a = take(hn * 4);
  z.vals_b = take(hn * 4);
  z.ranks = take(hn * 4);
  z.hist = take((size_t)heads * z.nblk_max * 256 * 4);
  z.new_len = take(hp * 4);
  z.flag = take(4);
  z.total = off;
  return z;
}

hipError_t run_diversity_score(const DivArgs& a, double* score_sum_host, int32_t* err_flag_host, hipStream_t s) {
  const DivK k = make_k(a);
  hipError_t e = enqueue_scores(a, k, s);
  if (e != hipSuccess) return e;
  return finish(a, k, nullptr, score_sum_host, err_flag_host, s);
}

hipError_t run_diversity_prune(const DivArgs& a, int32_t* new_len_host, double* score_sum_host,
                               int32_t* err_flag_host, hipStream_t s) {
  const DivSizes& z = a.sizes;
  const DivK k = make_k(a);
  hipError_t e = enqueue_scores(a, k, s);
  if (e != hipSuccess) return e;
  const int H = a.geom.heads;
  e = launch_rank_segments(reinterpret_cast<uint32_t*>(a.ws + z.keys_a), reinterpret_cast<uint32_t*>(a.ws + z.keys_b),
                           reinterpret_cast<uint32_t*>(a.ws + z.vals_a), reinterpret_cast<uint32_t*>(a.ws + z.vals_b),
                           reinterpret_cast<int32_t*>(a.ws + z.ranks), reinterpret_cast<uint32_t*>(a.ws + z.hist),
                           (int)a.N, H, k.flag, s);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)a.P, (unsigned)H);
  if (a.geom.esize == 2)
    div_compact_kernel<__bf16><<<grid, dim3(kThreads), 0, s>>>(k);
  else
    div_compact_kernel<float><<<grid, dim3(kThreads), 0, s>>>(k);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return finish(a, k, new_len_host, score_sum_host, err_flag_host, s);
}

}  // namespace kvs
