// Page write, page merge, page-table upload and per-head tables, gfx950.
//
// Page write (LingBot-Map 20 FPS explainer, "Page-Aligned Tensor Layout":
// a frame's tokens go straight into a page-aligned layout, no padding between
// frames, no extra copies).  A frame's K and V arrive as [T][H][D]; the page
// stores each as [H][Ts][D] (Ts = T rounded up to 64), plus the global token
// id of every slot.  One workgroup moves a 64-token block of one head: 128-byte
// rows (bf16) copied with 16-byte accesses on both sides.  Slots T..Ts-1 are
// zero-filled.  Each byte is touched once by this kernel, so loads and stores
// are nontemporal (streamed past the caches).

#include <hip/hip_runtime.h>

#include "blockscan.h"
#include "kernels.h"

namespace kvs {
namespace {

constexpr int D = kHeadDim;

// One workgroup: tokens t0..t0+63 of head h of one frame into one page.
template <typename T>
__device__ void append_block(const PageGeom& g, char* page, const T* __restrict__ k, const T* __restrict__ v,
                             int n_tokens, int64_t first_id, int h, int t0) {
  typedef int V16 __attribute__((ext_vector_type(4)));
  constexpr int VPR = D * sizeof(T) / 16;  // 16-byte vectors per row: 8 (bf16) or 16 (fp32)
  constexpr int RPP = 256 / VPR;           // rows per pass
  const int H = g.heads;
  const int tid = threadIdx.x;
  const int r = tid / VPR, c = tid % VPR;
  V16* kdst = reinterpret_cast<V16*>(page + g.k_off) + (int64_t)h * g.ts * VPR;
  V16* vdst = reinterpret_cast<V16*>(page + g.v_off) + (int64_t)h * g.ts * VPR;
  const V16* ksrc = reinterpret_cast<const V16*>(k);
  const V16* vsrc = reinterpret_cast<const V16*>(v);
  V16 kk[64 / RPP], vv[64 / RPP];
#pragma unroll
  for (int pp = 0; pp < 64 / RPP; ++pp) {
    const int t = t0 + r + RPP * pp;
    if (t < n_tokens) {
      kk[pp] = __builtin_nontemporal_load(&ksrc[((int64_t)t * H + h) * VPR + c]);
      vv[pp] = __builtin_nontemporal_load(&vsrc[((int64_t)t * H + h) * VPR + c]);
    } else {
      kk[pp] = V16{};
      vv[pp] = V16{};
    }
  }
#pragma unroll
  for (int pp = 0; pp < 64 / RPP; ++pp) {
    const int t = t0 + r + RPP * pp;
    __builtin_nontemporal_store(kk[pp], &kdst[(int64_t)t * VPR + c]);
    __builtin_nontemporal_store(vv[pp], &vdst[(int64_t)t * VPR + c]);
  }
  if (h == 0 && tid < 64) {
    const int t = t0 + tid;
    int32_t* ids = reinterpret_cast<int32_t*>(page + g.id_off);
    ids[t] = t < n_tokens ? (int32_t)(first_id + t) : -1;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void append_kernel(PageGeom g, char* page, const T* __restrict__ k,
                                                     const T* __restrict__ v, int n_tokens, int64_t first_id) {
  append_block<T>(g, page, k, v, n_tokens, first_id, blockIdx.y, blockIdx.x * 64);
}

// A frame's page write that also uploads (the first chunk of) a layer's
// attention table: the block after the page's 64-token blocks copies it.
template <typename T>
__global__ __launch_bounds__(256) void append_table_kernel(PageGeom g, char* page, const T* __restrict__ k,
                                                           const T* __restrict__ v, int n_tokens, int64_t first_id,
                                                           DevEntry* dst, TableChunk chunk) {
  if (blockIdx.x == gridDim.x - 1) {
    const int i = threadIdx.x;
    if (blockIdx.y == 0 && i < chunk.count) dst[chunk.first + i] = chunk.e[i];
    return;
  }
  append_block<T>(g, page, k, v, n_tokens, first_id, blockIdx.y, blockIdx.x * 64);
}

// Several layers' frames in one launch: blockIdx.z = layer within the chunk.
template <typename T>
__global__ __launch_bounds__(256) void append_layers_kernel(PageGeom g, char* pool, AppendLayers al,
                                                            const T* __restrict__ k, const T* __restrict__ v,
                                                            int n_tokens, int64_t first_id) {
  const int64_t frame_elems = (int64_t)n_tokens * g.heads * D;
  const int z = blockIdx.z;
  append_block<T>(g, pool + al.page_offset[z], k + z * frame_elems, v + z * frame_elems, n_tokens, first_id,
                  blockIdx.y, blockIdx.x * 64);
}

// Page merge: block (item, part) appends the rows of one head of K (part < H)
// or V (H <= part < 2H), or the token ids (part 2H), of page src after the
// dst_off rows already in page dst.  Source and destination are different
// pages, so every row moves independently.
template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(PageGeom g, char* pool, MergeChunk c) {
  typedef int V16 __attribute__((ext_vector_type(4)));
  constexpr int VPR = D * sizeof(T) / 16;  // 16-byte vectors per row
  constexpr int RPP = 256 / VPR;           // rows per pass
  const MergeItem it = c.item[blockIdx.x];
  const int part = blockIdx.y, H = g.heads, tid = threadIdx.x;
  const char* src = pool + it.src_offset;
  char* dst = pool + it.dst_offset;
  if (part < 2 * H) {
    const int h = part < H ? part : part - H;
    const int64_t off = (part < H ? g.k_off : g.v_off);
    const V16* s = reinterpret_cast<const V16*>(src + off) + (int64_t)h * g.ts * VPR;
    V16* d = reinterpret_cast<V16*>(dst + off) + ((int64_t)h * g.ts + it.dst_off) * VPR;
    const int r = tid / VPR, cc = tid % VPR;
    for (int r0 = 0; r0 < it.count; r0 += 4 * RPP) {
      V16 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = r0 + u * RPP + r;
        v[u] = row < it.count ? __builtin_nontemporal_load(&s[row * VPR + cc]) : V16{};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = r0 + u * RPP + r;
        if (row < it.count) __builtin_nontemporal_store(v[u], &d[row * VPR + cc]);
      }
    }
  } else {
    const int32_t* si = reinterpret_cast<const int32_t*>(src + g.id_off);
    int32_t* di = reinterpret_cast<int32_t*>(dst + g.id_off) + it.dst_off;
    for (int i = tid; i < it.count; i += 256) di[i] = si[i];
  }
}

// Per-head page merge: block (item, part) appends head h's rows of page src
// after the rows head h already holds in page dst, for K (part < H) or V
// (H <= part < 2H); part 2H writes the destination's new per-head lengths
// when this item is the last move into it.  Moves of one launch read pages
// that no move of it writes, and write disjoint row ranges.
template <typename T>
__global__ __launch_bounds__(256) void merge_heads_kernel(PageGeom g, char* pool, int32_t* hlen, HeadMergeChunk c) {
  typedef int V16 __attribute__((ext_vector_type(4)));
  constexpr int VPR = D * sizeof(T) / 16;  // 16-byte vectors per row
  constexpr int RPP = 256 / VPR;           // rows per pass
  const int it = blockIdx.x, part = blockIdx.y, H = g.heads, tid = threadIdx.x;
  if (part == 2 * H) {
    if (c.last[it])
      for (int h = tid; h < H; h += 256) {
        const int32_t* v = &c.hv[2 * (it * H + h)];
        hlen[(int64_t)c.dst_phys[it] * H + h] = v[0] + v[1];
      }
    return;
  }
  const int h = part < H ? part : part - H;
  const int off = c.hv[2 * (it * H + h)], count = c.hv[2 * (it * H + h) + 1];
  const int64_t seg = part < H ? g.k_off : g.v_off;
  const V16* src = reinterpret_cast<const V16*>(pool + c.src_offset[it] + seg) + (int64_t)h * g.ts * VPR;
  V16* dst = reinterpret_cast<V16*>(pool + c.dst_offset[it] + seg) + ((int64_t)h * g.ts + off) * VPR;
  const int r = tid / VPR, cc = tid % VPR;
  for (int r0 = 0; r0 < count; r0 += 4 * RPP) {
    V16 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = r0 + u * RPP + r;
      v[u] = row < count ? __builtin_nontemporal_load(&src[row * VPR + cc]) : V16{};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = r0 + u * RPP + r;
      if (row < count) __builtin_nontemporal_store(v[u], &dst[row * VPR + cc]);
    }
  }
}

__global__ void table_upload_kernel(DevEntry* dst, TableChunk chunk) {
  const int i = threadIdx.x;
  if (i < chunk.count) dst[chunk.first + i] = chunk.e[i];
}

// One workgroup per head: head h's table from the shared one.  An entry whose
// tile_start is nonzero takes its length from hlen[phys * H + h], any other
// keeps len; tile and token prefixes are rebuilt, and entry n (the sentinel)
// holds the head's totals.
__global__ __launch_bounds__(256) void head_tables_kernel(DevEntry* out, const DevEntry* base, int n,
                                                          const int32_t* hlen, int H) {
  __shared__ int32_t scan[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  DevEntry* t = out + (int64_t)h * (n + 1);
  const int per = (n + 255) / 256;
  const int b = min(tid * per, n), e = min(b + per, n);
  auto len_of = [&](const DevEntry& be) { return be.tile_start ? hlen[(int64_t)be.phys * H + h] : be.len; };
  int32_t tiles = 0, toks = 0;
  for (int i = b; i < e; ++i) {
    const int32_t len = len_of(base[i]);
    tiles += (len + kTile - 1) / kTile;
    toks += len;
  }
  int32_t tiles_tot = 0, toks_tot = 0;
  int32_t t0 = block_excl_scan<256>(tiles, scan, &tiles_tot);
  int32_t k0 = block_excl_scan<256>(toks, scan, &toks_tot);
  for (int i = b; i < e; ++i) {
    const DevEntry be = base[i];
    const int32_t len = len_of(be);
    t[i] = DevEntry{be.phys, len, t0, k0};
    t0 += (len + kTile - 1) / kTile;
    k0 += len;
  }
  if (tid == 0) t[n] = DevEntry{0, 0, tiles_tot, toks_tot};
}

}  // namespace

hipError_t launch_head_tables(DevEntry* out, const DevEntry* base, int n, const int32_t* hlen, int heads,
                              hipStream_t s) {
  head_tables_kernel<<<dim3((unsigned)heads), dim3(256), 0, s>>>(out, base, n, hlen, heads);
  return hipGetLastError();
}

hipError_t launch_append_layers(const PageGeom& g, char* pool, const AppendLayers& al, int n_layers,
                                const void* k, const void* v, int n_tokens, int64_t first_token_id,
                                hipStream_t s) {
  dim3 grid((unsigned)(g.ts / 64), (unsigned)g.heads, (unsigned)n_layers);
  if (g.esize == 2)
    append_layers_kernel<__bf16><<<grid, dim3(256), 0, s>>>(g, pool, al, static_cast<const __bf16*>(k),
                                                             static_cast<const __bf16*>(v), n_tokens, first_token_id);
  else
    append_layers_kernel<float><<<grid, dim3(256), 0, s>>>(g, pool, al, static_cast<const float*>(k),
                                                            static_cast<const float*>(v), n_tokens, first_token_id);
  return hipGetLastError();
}

hipError_t launch_merge(const PageGeom& g, char* pool, const MergeChunk& c, hipStream_t s) {
  if (c.n <= 0) return hipSuccess;
  dim3 grid((unsigned)c.n, (unsigned)(2 * g.heads + 1));
  if (g.esize == 2)
    merge_kernel<__bf16><<<grid, dim3(256), 0, s>>>(g, pool, c);
  else
    merge_kernel<float><<<grid, dim3(256), 0, s>>>(g, pool, c);
  return hipGetLastError();
}

hipError_t launch_head_merge(const PageGeom& g, char* pool, int32_t* hlen, const HeadMergeChunk& c, hipStream_t s) {
  if (c.n < 1) return hipSuccess;
  dim3 grid((unsigned)c.n, (unsigned)(2 * g.heads + 1));
  if (g.esize == 2)
    merge_heads_kernel<__bf16><<<grid, dim3(256), 0, s>>>(g, pool, hlen, c);
  else
    merge_heads_kernel<float><<<grid, dim3(256), 0, s>>>(g, pool, hlen, c);
  return hipGetLastError();
}

hipError_t launch_table_upload(DevEntry* dst, const DevEntry* src, int n, hipStream_t s) {
  for (int first = 0; first < n; first += kUploadChunk) {
    TableChunk c;
    c.first = first;
    c.count = n - first < kUploadChunk ? n - first : kUploadChunk;
    for (int i = 0; i < c.count; ++i) c.e[i] = src[first + i];
    table_upload_kernel<<<dim3(1), dim3(kUploadChunk), 0, s>>>(dst, c);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_append_table(const PageGeom& g, char* page, const void* k, const void* v, int n_tokens,
                               int64_t first_token_id, DevEntry* dst, const DevEntry* src, int n, hipStream_t s) {
  TableChunk c;
  c.first = 0;
  c.count = n < kUploadChunk ? n : kUploadChunk;
  for (int i = 0; i < c.count; ++i) c.e[i] = src[i];
  dim3 grid((unsigned)(g.ts / 64 + 1), (unsigned)g.heads);
  if (g.esize == 2)
    append_table_kernel<__bf16><<<grid, dim3(256), 0, s>>>(g, page, static_cast<const __bf16*>(k),
                                                            static_cast<const __bf16*>(v), n_tokens, first_token_id,
                                                            dst, c);
  else
    append_table_kernel<float><<<grid, dim3(256), 0, s>>>(g, page, static_cast<const float*>(k),
                                                           static_cast<const float*>(v), n_tokens, first_token_id,
                                                           dst, c);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n <= kUploadChunk) return err;
  return launch_table_upload(dst + kUploadChunk, src + kUploadChunk, n - kUploadChunk, s);
}

hipError_t launch_append(const PageGeom& g, char* page, const void* k, const void* v, int n_tokens,
                         int64_t first_token_id, hipStream_t s) {
  dim3 grid((unsigned)(g.ts / 64), (unsigned)g.heads);
  if (g.esize == 2)
    append_kernel<__bf16><<<grid, dim3(256), 0, s>>>(g, page, static_cast<const __bf16*>(k),
                                                      static_cast<const __bf16*>(v), n_tokens, first_token_id);
  else
    append_kernel<float><<<grid, dim3(256), 0, s>>>(g, page, static_cast<const float*>(k),
                                                     static_cast<const float*>(v), n_tokens, first_token_id);
  return hipGetLastError();
}

}  // namespace kvs
