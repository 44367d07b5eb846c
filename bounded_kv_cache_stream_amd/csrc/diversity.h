// Internal interface of the diversity-scored per-head pruning pipeline.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "kernels.h"

namespace kvs {

constexpr int32_t kDivErrNan = 1;  // a key is not finite (its score is NaN)

// Byte offsets of the diversity buffers inside its workspace region.
struct DivSizes {
  int64_t n_max;  // candidates per head
  int32_t p_max, h_max, nblk_max;
  size_t entries, partial, mean, spart, total_sum, keys_a, keys_b, vals_a, vals_b, ranks, hist, new_len, flag,
      total;
};

DivSizes div_sizes(int64_t n_max, int32_t p_max, int32_t heads);

struct DivArgs {
  char* ws;  // start of the diversity workspace region
  DivSizes sizes;
  char* pool;
  PageGeom geom;
  // The layer's candidate pages, in table order: phys = physical page, len =
  // rows of every head, tile_start != 0 when the page's per-head lengths are
  // in hlen_dev (see launch_head_tables); P of them.
  const DevEntry* base_host;
  int32_t P;
  int32_t* hlen_dev;  // [physical page][heads] per-head lengths; the prune writes its pages' new lengths
  int64_t N;          // the largest per-head candidate count
  int64_t keep;       // candidates kept per head (prune only)
  float* scores_out;  // optional [heads][score_stride], candidate order
  int64_t score_stride;
};

// Scores every candidate of every head; waits, and returns the sum of the
// float64 scores over heads and candidates, and the error flags.
hipError_t run_diversity_score(const DivArgs& a, double* score_sum_host, int32_t* err_flag_host, hipStream_t s);

// Scores, keeps each head's `keep` most diverse candidates and compacts every
// page and head in place; waits, and returns the new lengths ([P][heads]),
// the score sum before the prune, and the error flags (on an error nothing
// moves).
hipError_t run_diversity_prune(const DivArgs& a, int32_t* new_len_host, double* score_sum_host,
                               int32_t* err_flag_host, hipStream_t s);

}  // namespace kvs
