// Internal interface between the C-ABI runtime (kvstream.cpp) and the HIP
// kernels (*.hip).  Not installed; callers use include/kvstream.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace kvs {

constexpr int kHeadDim = 64;
constexpr int kTile = 64;  // KV tile (tokens) of the attention kernel, and page-stride unit
constexpr int kAttendRows = 256;  // query rows per attention workgroup

// One entry of the device copy of a layer's attended table.
struct DevEntry {
  int32_t phys;        // physical page index in the pool
  int32_t len;         // valid tokens
  int32_t tile_start;  // number of kTile tiles in the entries before this one
  int32_t tok_start;   // number of tokens in the entries before this one
};

// Geometry of one page (bytes), see kv_pool_layout in include/kvstream.h.
struct PageGeom {
  int64_t page_bytes;
  int64_t k_off, v_off, id_off;
  int32_t ts;    // token stride
  int32_t heads;
  int32_t esize; // 2 (bf16) or 4 (fp32)
};

constexpr int kUploadChunk = 192;
struct TableChunk {
  int32_t first;
  int32_t count;
  DevEntry e[kUploadChunk];
};

hipError_t launch_table_upload(DevEntry* dst, const DevEntry* src, int n, hipStream_t s);

// Per-head tables out[h][0..n] (stride n + 1) from the shared table base[n]:
// an entry with tile_start != 0 holds hlen[phys * heads + h] rows of head h,
// any other holds len in every head; tile_start / tok_start are rebuilt per
// head and entry n of each holds the head's tile and token totals.
hipError_t launch_head_tables(DevEntry* out, const DevEntry* base, int n, const int32_t* hlen, int heads,
                              hipStream_t s);

hipError_t launch_append(const PageGeom& g, char* page, const void* k, const void* v, int n_tokens,
                         int64_t first_token_id, hipStream_t s);

// launch_append and launch_table_upload(dst, src, n) in one launch (table
// entries past the first kUploadChunk go in further upload launches).
hipError_t launch_append_table(const PageGeom& g, char* page, const void* k, const void* v, int n_tokens,
                               int64_t first_token_id, DevEntry* dst, const DevEntry* src, int n, hipStream_t s);

// Destination pages of one multi-layer append launch (byte offsets into the pool).
constexpr int kAppendLayersChunk = 128;
struct AppendLayers {
  int64_t page_offset[kAppendLayersChunk];
};
// k, v: [n_layers][n_tokens][H][D]; n_layers <= kAppendLayersChunk.
hipError_t launch_append_layers(const PageGeom& g, char* pool, const AppendLayers& al, int n_layers,
                                const void* k, const void* v, int n_tokens, int64_t first_token_id,
                                hipStream_t s);

// Page merges of one launch: item i moves count tokens (all heads of K and V,
// and their ids) from the start of page src to slots dst_off.. of page dst
// (byte offsets of the pages in the pool).
constexpr int kMergeChunk = 128;
struct MergeItem {
  int64_t src_offset, dst_offset;
  int32_t dst_off, count;
};
struct MergeChunk {
  int32_t n;
  MergeItem item[kMergeChunk];
};
hipError_t launch_merge(const PageGeom& g, char* pool, const MergeChunk& c, hipStream_t s);

// Per-head page merges of one launch (pages whose heads hold different rows):
// item i moves, for every head h, rows 0 .. count-1 of head h of page src to
// slots off.. of head h of page dst, with (off, count) = hv[2*(i*heads+h)],
// hv[2*(i*heads+h)+1]; an item with last = 1 also writes off + count, the
// page's new per-head lengths, to hlen[dst_phys * heads + h].  Token ids are
// not moved (a pruned page's id row describes none of its heads).
constexpr int kHeadMergeItems = 16;
constexpr int kHeadMergeInts = 640;
struct HeadMergeChunk {
  int32_t n;
  int64_t src_offset[kHeadMergeItems], dst_offset[kHeadMergeItems];
  int32_t dst_phys[kHeadMergeItems];
  int32_t last[kHeadMergeItems];
  int32_t hv[kHeadMergeInts];
};
hipError_t launch_head_merge(const PageGeom& g, char* pool, int32_t* hlen, const HeadMergeChunk& c, hipStream_t s);

struct AttendParams {
  const void* q;
  void* out;
  float* lse;
  float* part_o;   // [splits][n_q][H][D] fp32 (splits > 1)
  float* part_ml;  // [splits][n_q][H][2] fp32 (splits > 1)
  const char* pool;
  const DevEntry* table;
  int32_t n_entries;
  int32_t total_tiles;   // per-page tiles of the shared table
  int32_t total_tokens;  // tokens of the shared table
  // 0: one table for every head.  Otherwise head h's table starts at
  // table + h * head_stride (n_entries entries, zero-length where the head
  // holds nothing of that page) and entry n_entries of it holds the head's
  // per-page tile count in tile_start and token count in tok_start.
  int32_t head_stride;
  int32_t packed;  // 1: tiles packed over each head's token sequence, 0: tiles per page
  int32_t inline_table;  // 1: the shared table rides in the launch's TableChunk argument, not in table
  int32_t splits;
  int32_t n_q;
  float scale_log2;  // sm_scale * log2(e)
};

// ev_start / ev_stop (optional): recorded on s right before and right after
// the attention kernel (before the split-KV combine).
// inl (bf16 only, with p.inline_table set): a shared table of at most
// kUploadChunk entries passed by value in the kernel's arguments, which saves
// the table-upload launch.
hipError_t launch_attend(const PageGeom& g, const AttendParams& p, bool bf16, hipStream_t s,
                         hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
                         const TableChunk* inl = nullptr);

// Device scratch of the allocation-free attention entry point: a file-scope
// array in attend.hip, one copy per GPU, holding the split-KV partials.
constexpr size_t kAttendScratchBytes = size_t(64) << 20;
constexpr int kAttendScratchDevices = 64;
// This GPU's copy (the current device): its address is looked up once per
// device and kept.
hipError_t attend_scratch_address(char** out);

}  // namespace kvs
