// Internal interface of the diversity-scored per-head pruning pipeline.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "kernels.h"

namespace kvs {

constexpr int32_t kDivErrNan = 1;  // a key is not finite (its score is NaN)

// One layer of a call (device copy, one per slot).
struct DivLayer {
  int64_t keys_off;  // the layer's keys start at key store + keys_off: [H][N]
  int64_t N;         // key stride per head: at least the layer's largest candidate count
  int64_t keep;      // candidates kept per head (prune)
  int32_t P;         // candidate pages
  int32_t rescore;   // 1: score the layer in this call
  int32_t layer;     // the pool layer (indexes the per-layer first-digit histograms)
  int32_t pad;
};

// Byte offsets of the diversity buffers inside its workspace region, sized
// for `layers` slots (one per layer of a call).  params and bases are one
// contiguous block that the host fills with a single copy.
struct DivSizes {
  int64_t n_max;  // candidates per head
  int32_t p_max, h_max, layers;
  size_t params, bases, tabs, partial, mean, spart, totals, flags, dstate, lt_cnt, eq_cnt, hist0, hcount, kept,
      new_len, total;
};

DivSizes div_sizes(int64_t n_max, int32_t p_max, int32_t heads, int32_t layers);

// Host layout of the params + bases block for n slots: DivLayer [n] at 0,
// then candidate pages [n][p_max] at bases - params (phys = physical page,
// len = rows of every head, tile_start != 0 when the page's per-head lengths
// are in the head-length array).
size_t div_staging_bytes(const DivSizes& z, int n);
inline DivLayer* div_staging_layers(char* staging) { return reinterpret_cast<DivLayer*>(staging); }
inline DevEntry* div_staging_bases(const DivSizes& z, char* staging, int slot) {
  return reinterpret_cast<DevEntry*>(staging + (z.bases - z.params)) + (int64_t)slot * z.p_max;
}

struct DivCall {
  char* ws;  // start of the diversity workspace region
  DivSizes sizes;
  char* pool;
  PageGeom geom;
  int32_t* hlen_dev;      // [physical page][heads] per-head lengths; a prune writes its pages' new lengths
  uint32_t* keys_dev;     // the key store (each layer's keys at its keys_off: per head a high plane, then a low plane)
  const char* staging;    // device address of the pinned host block of div_staging_bytes(sizes, n) bytes
  int32_t n;              // slots
  int32_t max_P;          // the largest P over the slots
  int64_t max_N;          // the largest N over the slots
  bool any_rescore;       // some slot scores
  bool prune;             // select and compact after the scoring
  double* scores_out;     // optional [heads][score_stride] of slot 0, candidate order
  int64_t score_stride;
};

// Enqueues one call: the per-head candidate tables of every slot, the
// scoring of the slots with rescore (keys into the key store, the float64
// score sum into the totals), and for a prune the per-head top-K and the
// compaction of every page and head.  Error flags: one word per slot, then
// one for the call; no row moves once the call's word is set.
hipError_t enqueue_diversity(const DivCall& c, hipStream_t s);

// Device addresses of the outputs the host reads back: totals, then flags,
// then the new lengths [slot][p_max][heads], adjacent in that order.
inline double* div_totals(const DivCall& c) { return reinterpret_cast<double*>(c.ws + c.sizes.totals); }
inline int32_t* div_flags(const DivCall& c) { return reinterpret_cast<int32_t*>(c.ws + c.sizes.flags); }

}  // namespace kvs
