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
constexpr int32_t kRankTile = 2048;    // keys per rank block (sorted by one workgroup)
constexpr int32_t kRankGroups = 8;     // most groups of blocks a key is counted against
constexpr int32_t kRankParts = 1 + kRankGroups;  // count slices per ranked segment
// Largest segments x blocks^2 ranked by block sort + counts (their search work
// grows as N x blocks); beyond it the radix passes, whose cost is nearly flat
// in N, are faster.
constexpr int64_t kSortCountMax = 12000;
constexpr int32_t kMaxPageTokensScored = 8192;
constexpr int kMaxWindow = 8;          // largest CLCES layer window
constexpr int kSelBits = 11;           // bits of the select digits (the last pass takes the 9 left)
constexpr int kSelPasses = 6;

// Ranks of one step's window slots, int32 [N] each: a slot ranked in an
// earlier step reads w[slot]; a slot ranked in this step has n_part count
// slices of N at part[slot] (stride N) whose sum is its rank, stored at
// dst[slot] for later steps.
struct RankIn {
  const int32_t* w[kMaxWindow];
  const int32_t* part[kMaxWindow];
  int32_t* dst[kMaxWindow];
  int32_t n_part;
};

// Byte offsets of the CLCES buffers inside its workspace region.
struct ClcesSizes {
  int64_t n_max;
  int32_t p_max, w_max;
  size_t keys, keys_b, vals_a, vals_b, blk_cnt, sorted, sorted_idx, part, scur, shat, sel_hist, sel_state, list, list_cnt, entries, counts,
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
  // per window slot (oldest first): where the layer's ranks are (rank_new =
  // 0: from an earlier step) or go (rank_new = 1: ranked in this step)
  int32_t* rank_dst[kMaxWindow];
  uint8_t rank_new[kMaxWindow];
  int32_t n_rank;      // slots with rank_new set
  bool rank_radix;     // rank by the radix passes whatever the size
  double* s_hat_out;   // optional float64 [N]
  // optional: one word per page in host-visible memory (device address),
  // written by the index step as soon as the page's new length is known, so
  // that a waiting host can go on while the rows still move:
  // (slot_seq << 32) | new length, or (slot_seq << 32) | kSlotError | flag
  unsigned long long* host_slots;
  uint32_t slot_seq;
};

constexpr uint32_t kSlotError = 0x80000000u;

// Stable ascending rank of every key within each of `segments` segments of N
// keys (keys: [segments][N]) as count slices whose sum is the rank: the blocks
// of kRankTile keys are sorted (sorted, sorted_idx: [segments][whole blocks]),
// each key's rank within its block goes to slice 0 of part
// ([segments][kRankParts][N]) and its counts against the other blocks to the
// next slices.  Returns the number of slices written per segment through
// *n_part.
hipError_t launch_rank_sort_count(const uint32_t* keys, uint32_t* sorted, uint32_t* sorted_idx, int32_t* part, int N,
                                  int segments, const int32_t* flag, int* n_part, hipStream_t s);
// The same ranks by 4 LSD radix passes of 8 bits (two launches each; keys_a
// is overwritten), written to dst[w] ([N] each).
hipError_t launch_rank_radix(uint32_t* keys_a, uint32_t* keys_b, uint32_t* vals_a, uint32_t* vals_b, uint32_t* blk_cnt,
                             int32_t* const* dst, int N, int segments, const int32_t* flag, hipStream_t s);

// Enqueues the whole step (kernels only, no wait).  Its result (the
// error flag, then the new length of each of the n_entries pages) is at
// clces_result(a) on the device once the stream reaches this point, until the
// next step that uses the same workspace.
hipError_t enqueue_clces(const ClcesArgs& a, hipStream_t s);
int32_t* clces_result(const ClcesArgs& a);

}  // namespace kvs
