// Workgroup-wide helpers shared by the scoring and compaction kernels: an
// exclusive scan and a digit histogram in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

// Exclusive scan of one value per thread over a workgroup of NT threads
// (lds: NT ints); *total, if given, receives the sum.  Every thread calls it.
template <int NT>
__device__ int32_t block_excl_scan(int32_t v, int32_t* lds, int32_t* total) {
  const int tid = threadIdx.x;
  lds[tid] = v;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    int32_t t = tid >= off ? lds[tid - off] : 0;
    __syncthreads();
    lds[tid] += t;
    __syncthreads();
  }
  const int32_t incl = lds[tid];
  if (total) *total = lds[NT - 1];
  __syncthreads();
  return incl - v;
}

// Add one to cnt[d] for every active lane with `valid`, aggregating lanes of
// the wave that share the first lane's digit into one atomic (digits are often
// nearly uniform: the top bytes of similar floats).
__device__ inline void hist_add(uint32_t* cnt, uint32_t d, bool valid) {
  const unsigned long long act = __ballot(valid);
  if (act == 0) return;
  const int first = __ffsll((long long)act) - 1;
  const uint32_t lead = __shfl(d, first, 64);
  const unsigned long long same = __ballot(valid && d == lead);
  if ((threadIdx.x & 63) == first) atomicAdd(&cnt[lead], (uint32_t)__popcll(same));
  if (valid && d != lead) atomicAdd(&cnt[d], 1u);
}

}  // namespace kvs
