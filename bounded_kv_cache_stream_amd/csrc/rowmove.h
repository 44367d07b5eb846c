// In-page row moves shared by the compaction kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

typedef int V16 __attribute__((ext_vector_type(4)));  // a native vector: a struct copy would go through scratch

// Move the rows of one head of one page ([slot][d], 64 * sizeof(T) bytes each)
// from the move sources to the move destinations.  8 threads per row and 4
// vectors per thread (bf16): one pass of a 1024-thread workgroup moves 512
// rows, all loads issued before the stores.  Sources and destinations are
// disjoint (kept slots at or past a page's new length fill the holes below
// it), so no barrier is needed; the rows are touched once, so accesses are
// nontemporal.
template <typename T, int NT>
__device__ inline void move_rows(V16* rows, const uint16_t* src, const uint16_t* dst, int nm, int tid) {
  constexpr int VPR = 64 * sizeof(T) / 16;  // vectors per row
  constexpr int TPR = 8;                    // threads per row
  constexpr int UPR = VPR / TPR;            // vectors per thread per row
  constexpr int G = 4 / UPR;                // row groups per pass
  constexpr int RPP = NT / TPR;             // rows per group
  const int r = tid / TPR, c = tid % TPR;
  for (int i0 = 0; i0 < nm; i0 += RPP * G) {
    V16 v[G][UPR];
    int s[G], d[G];
#pragma unroll
    for (int gq = 0; gq < G; ++gq) {
      const int i = i0 + gq * RPP + r;
      s[gq] = i < nm ? src[i] : 0;  // past the end: load slot 0 (in bounds, never stored)
      d[gq] = i < nm ? dst[i] : -1;
    }
#pragma unroll
    for (int gq = 0; gq < G; ++gq)
#pragma unroll
      for (int u = 0; u < UPR; ++u) v[gq][u] = __builtin_nontemporal_load(&rows[s[gq] * VPR + c + TPR * u]);
#pragma unroll
    for (int gq = 0; gq < G; ++gq)
      if (d[gq] >= 0)
#pragma unroll
        for (int u = 0; u < UPR; ++u) __builtin_nontemporal_store(v[gq][u], &rows[d[gq] * VPR + c + TPR * u]);
  }
}

}  // namespace kvs
