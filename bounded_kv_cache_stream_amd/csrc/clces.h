// Internal interface of the CLCES scoring + top-k + compaction pipeline.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "kernels.h"

namespace kvs {

constexpr int32_t kClcesErrNan = 1;    // a raw score is NaN or negative
constexpr int32_t kClcesErrRow = 2;    // a token id is outside the score table
constexpr int32_t kClcesErrCount = 4;  // a page's kept count disagrees with its planned length
constexpr int32_t kRankTile = 512;     // keys per radix-sort workgroup
constexpr int32_t kMaxPageTokensScored = 8192;

// Byte offsets of the CLCES buffers inside its workspace region.
struct ClcesSizes {
  int64_t n_max;
  int32_t p_max, w_max, nblk_max;
  size_t keys_a, keys_b, vals_a, vals_b, ranks, scur, shat, hist, sel_hist, sel_state, entries, counts,
      move_src, move_dst, n_moves, flag, total;
};

ClcesSizes clces_sizes(int64_t n_max, int32_t p_max, int32_t w_max, int32_t ts_max);

struct ClcesArgs {
  char* ws;  // start of the CLCES workspace region
  ClcesSizes sizes;
  char* pool;
  PageGeom geom;
  const DevEntry* entries_host;  // candidate pages (phys, len, tok_start)
  int32_t n_entries;
  int32_t n_tokens;
  const float* score_table;
  int64_t score_rows;
  int32_t score_cols;
  int32_t first_layer;  // oldest window layer
  int32_t n_window;
  double lambda;
  int64_t keep;
  int32_t* keep_ids_out;
  int32_t* ranks_out;
};

// Stable ascending rank of every key within each of `segments` segments of N
// keys (keys_a: [segments][N], overwritten; ranks: [segments][N]), 4 LSD
// passes of 8 bits.  counts holds rank_counters(N, segments) counters; its
// first part (the chunk sums, which accumulate with atomics) is set to zero
// beforehand by the caller's first kernel.
int64_t rank_counters(int N, int segments);
hipError_t launch_rank_segments(uint32_t* keys_a, uint32_t* keys_b, uint32_t* vals_a, uint32_t* vals_b, int32_t* ranks,
                                uint32_t* counts, int N, int segments, const int32_t* flag, hipStream_t s);

// Enqueues the whole step, then waits for it and returns the new page
// lengths (one per candidate entry) and the error flags.
hipError_t run_clces(const ClcesArgs& a, int32_t* new_lens_host, int32_t* err_flag_host, hipStream_t s);

// The same step without the wait: enqueues the kernels only.  Its result (the
// error flag, then the new length of each of the n_entries pages) is at
// clces_result(a) on the device once the stream reaches this point, until the
// next step that uses the same workspace.
hipError_t enqueue_clces(const ClcesArgs& a, hipStream_t s);
int32_t* clces_result(const ClcesArgs& a);

}  // namespace kvs
