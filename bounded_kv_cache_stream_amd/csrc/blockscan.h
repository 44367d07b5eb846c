// Workgroup-wide exclusive scan shared by the compaction kernels.
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

}  // namespace kvs
