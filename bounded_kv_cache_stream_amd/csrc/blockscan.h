// Workgroup-wide helpers shared by the scoring and compaction kernels: an
// exclusive scan and a digit histogram in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

// Exclusive scan of one value per thread over a workgroup of NT threads
// (NT a multiple of 64; lds: at least NT / 64 ints); *total, if given,
// receives the sum.  Every thread calls it.  Each wave scans its lanes with
// shuffles, then the waves' sums go through LDS (two barriers in all).
template <int NT>
__device__ int32_t block_excl_scan(int32_t v, int32_t* lds, int32_t* total) {
  static_assert(NT % 64 == 0, "whole waves");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) lds[wave] = incl;
  __syncthreads();
  int32_t before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int32_t s = lds[w];
    before += w < wave ? s : 0;
    sum += s;
  }
  if (total) *total = sum;
  __syncthreads();  // lds may be rewritten by the next call
  return before + incl - v;
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
