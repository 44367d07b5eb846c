// Frame-to-cache attention over a paged KV cache, gfx950.
//
// Computes, per query row i and head h, softmax(sm_scale * q_i . k_j) v_j over
// every token j of a layer's attended page list (GCTStream explainer,
// "Frame-by-Frame Causal Processing": each new frame attends to the cached
// keys/values of earlier frames; "Scale-Frame Phase": the first frames attend
// to each other).  No token mask: a frame sees all of its own tokens.
//
// bf16 path (the hot one): flash-style online softmax with both contractions
// on MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation.
//   * workgroup = 4 waves = 256 query rows of one head; each wave owns two
//     32-row query blocks, so every K or V operand read from LDS feeds two
//     MFMAs (LDS reads, LDS staging and HBM->LDS traffic per flop are halved
//     against one block per wave);
//   * KV streamed in 64-token tiles, double-buffered in LDS with the next
//     tile's global loads in flight during the current tile (the next tile
//     is staged into LDS between the QK and PV products); K and V are both
//     [key][d] in the page and in LDS.  The K operand is one 16-byte LDS read;
//     the V^T operand of the PV product (8 consecutive keys of one d per lane)
//     comes from two ds_read_b64_tr_b16 transposing reads: within each group
//     of 16 lanes, lane i receives element i%4 of the 8-byte pieces addressed
//     by lanes 4j + i/4 (j = 0..3), so lanes that address 4 key rows x 16
//     columns receive 4 keys of one column each;
//   * scores are computed transposed, S^T = K Q^T, so each lane's accumulator
//     column is one query: the row max needs one cross-lane exchange (lane l
//     with l^32), the O rescale is lane-local, and the accumulator registers
//     are directly the B operand of O^T += V^T P^T.  For that, the A-operand
//     row m of the K read is taken from key pi(m) with
//     pi(m) = 16*(m>>4) + 8*((m>>2)&1) + 4*((m>>3)&1) + (m&3), which makes the
//     8 probabilities a lane holds for one 16-key MFMA step 8 consecutive keys;
//   * online softmax in the log2 domain (exp2 on v_exp_f32) without a per-tile
//     max: probabilities are taken against the running max, and the tile's
//     row sum (v_dot2_f32_bf16 over the same bf16 probabilities that enter the
//     PV MFMA) flags a tile whose largest probability would pass 2^16 (and the
//     first tile, whose max is still -inf).  Only such a tile takes its max,
//     raises the running max, rescales O and l and is redone.  On gfx950 VALU
//     work does not overlap MFMA work on a SIMD, so every VALU instruction
//     taken out of the tile loop is time saved;
//   * KV tiles per page (a page's last tile partial), or packed over each
//     head's token sequence (its pages' tokens in table order): a tile may
//     span page ends and only the sequence's last tile is partial, which
//     evens out per-head tables whose heads spread equal token counts over
//     their pages differently.  The page table is walked with scalar loads
//     (constant address space);
//   * the KV axis is split across workgroups (split-KV); partial (O, m, l) are
//     merged by attend_combine.  Workgroup ids are remapped so that all query
//     tiles of one (head, split) land on the same XCD and share its L2.
// fp32 path: one wave per (query, head), lanes over d -- a plain reference-
// grade kernel for fp32 caches.

#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace kvs {

// Split-KV partials of stream_attend_scratch, one copy per GPU, held until the
// process ends.  In host code this name is a host-side stand-in, never a
// device address: kernels get each GPU's copy from attend_scratch_address.
static __device__ __align__(256) char scratch[kAttendScratchBytes];

namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int D = kHeadDim;
constexpr int BN = kTile;    // keys per tile
constexpr int BM = kAttendRows;  // query rows per workgroup (4 waves x 64)
constexpr int LDS_LD = 72;   // bf16 per LDS row (64 + 8 pad)
constexpr float kLn2 = 0.69314718055994530942f;

// Transposing LDS read (ds_read_b64_tr_b16) of four bf16.
__device__ inline bf16x4 lds_read_tr4(const bf16* p) {
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ inline int perm_key(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}

// Bijective XCD-aware remap: consecutive logical ids land on one XCD.
__device__ inline int xcd_remap(int bid, int nwg) {
  const int nx = 8;
  int xcd = bid % nx, round = bid / nx;
  int base = nwg / nx, extra = nwg % nx;
  int start = xcd * base + (xcd < extra ? xcd : extra);
  return start + round;
}

__device__ inline float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// two waves per SIMD: 256 VGPRs per lane for the two query blocks' accumulators
// PACKED: tiles over each head's token sequence (a tile may span page ends),
// else tiles per page (a page's last tile is partial).
template <bool PACKED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attend_bf16_kernel(PageGeom g, AttendParams p, int qtiles,
                                                                                              const TableChunk inl) {
  constexpr int RPP = 32;          // K/V rows staged per pass (8 threads per 128-byte row)
  constexpr int PP = BN / RPP;     // passes per tile
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BN * LDS_LD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BN * LDS_LD];

  const int H = g.heads;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = logical % qtiles;
  const int rest = logical / qtiles;
  const int sp = rest % p.splits;
  const int h = rest / p.splits;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int ql = lane & 31;
  const int grp = lane >> 5;
  // each wave owns two 32-row query blocks
  int qrow[2];
  bool qvalid[2];
  const bf16* q = static_cast<const bf16*>(p.q);
  bf16x8 qf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qrow[qb] = qt * BM + wave * 64 + qb * 32 + ql;
    qvalid[qb] = qrow[qb] < p.n_q;
    if (qvalid[qb]) {
      const bf16x8* src = reinterpret_cast<const bf16x8*>(q + ((int64_t)qrow[qb] * H + h) * D);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[qb][ks] = src[2 * ks + grp];
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[qb][ks] = bf16x8{};
    }
  }

  // The page table is read-only for the kernel's lifetime: read it through the
  // constant address space so that the walk over it runs on scalar loads and
  // SALU.  A short shared table comes in the kernel's own arguments (the
  // kernarg segment is constant memory too).
  typedef const __attribute__((address_space(4))) DevEntry* ConstTable;
  const ConstTable tab = p.inline_table ? (ConstTable)&inl.e[0] : (ConstTable)(p.table + (int64_t)h * p.head_stride);
  // Packed: tile t holds tokens 64t .. 64t+63 of the head's token sequence
  // (the entries' tokens in table order) whatever pages they are in, so only
  // the sequence's last tile is partial.  Per page: the tiles of entry e are
  // tile_start .. tile_start + ceil(len / 64) - 1.
  const int total_tokens = p.head_stride ? tab[p.n_entries].tok_start : p.total_tokens;
  const int total_tiles = PACKED ? (total_tokens + BN - 1) / BN
                                 : (p.head_stride ? tab[p.n_entries].tile_start : p.total_tiles);
  const int t_begin = (int)((int64_t)sp * total_tiles / p.splits);
  const int t_end = (int)((int64_t)(sp + 1) * total_tiles / p.splits);

  // e: the entry of the next tile to load.  Packed: the entry holding token
  // 64 t, the last entry whose tok_start is at most that token (entries before
  // it that start at the same token are empty).  Per page: the last entry
  // whose first tile is at most t.
  int e = 0;
  {
    const int j = PACKED ? t_begin * BN : t_begin;
    int lo = 0, hi = p.n_entries - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if ((PACKED ? tab[mid].tok_start : tab[mid].tile_start) <= j) lo = mid; else hi = mid - 1;
    }
    e = lo;
  }

  f32x16 oacc[2][2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int i = 0; i < 16; ++i) { oacc[qb][0][i] = 0.f; oacc[qb][1][i] = 0.f; }
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const int lrow = tid >> 3;
  const int lchunk = tid & 7;
  const int64_t head_off = (int64_t)h * g.ts * D;
  const int64_t head_off_bytes = head_off * (int64_t)sizeof(bf16);
  // Packed: entry e's first token and end, and the address of its head's
  // first row, with the same for the next entry that holds tokens (len 0:
  // none), kept in SGPRs and reloaded only when the walk enters the next
  // entry (once per page, not per tile)
  int e_tok = 0, e_end = 0, n_len = 0;
  const char* e_rows = nullptr;
  const char* n_rows = nullptr;
  auto enter = [&]() {
    e_tok = tab[e].tok_start;
    e_end = e_tok + tab[e].len;
    e_rows = p.pool + (int64_t)tab[e].phys * g.page_bytes + head_off_bytes;
    int e2 = e + 1;
    while (e2 < p.n_entries && tab[e2].len == 0) ++e2;
    n_len = e2 < p.n_entries ? tab[e2].len : 0;
    n_rows = e2 < p.n_entries ? p.pool + (int64_t)tab[e2].phys * g.page_bytes + head_off_bytes : e_rows;
  };
  if constexpr (PACKED) enter();

  bf16x8 kreg[PP], vreg[PP];
  const uint32_t lane_off = (uint32_t)((lrow * D + lchunk * 8) * sizeof(bf16));
  // Tile rows of this thread: lrow + RPP * pp.  Per page: the tile's rows
  // are consecutive rows of its page (address in SGPRs plus the lane's
  // constant offset; a page's last tile reads up to the token stride, a
  // multiple of 64).  Packed: a full tile inside one page (most tiles) loads
  // the same way.  Otherwise the entries the tile spans
  // are walked with scalar loads, one segment of consecutive tile rows per
  // entry, and each row's byte offset from the pool comes from its segment;
  // rows past the last token read row 0 of the tile (their V rows are zeroed
  // and their scores masked).
  auto load_tile = [&](int t) -> int {
    if constexpr (!PACKED) {
      while (t >= tab[e].tile_start + ((tab[e].len + BN - 1) / BN)) ++e;
      const int row0 = (t - tab[e].tile_start) * BN;
      const int nvalid = min(BN, tab[e].len - row0);
      const char* base =
          p.pool + (int64_t)tab[e].phys * g.page_bytes + (head_off + (int64_t)row0 * D) * (int64_t)sizeof(bf16);
      const char* kt = base + g.k_off;
      const char* vt = base + g.v_off;
#pragma unroll
      for (int pp = 0; pp < PP; ++pp) {
        kreg[pp] = *reinterpret_cast<const bf16x8*>(kt + lane_off + pp * RPP * D * sizeof(bf16));
        vreg[pp] = *reinterpret_cast<const bf16x8*>(vt + lane_off + pp * RPP * D * sizeof(bf16));
      }
      return nvalid;
    }
    const int j0 = t * BN;
    // the entry holding token j0: entries are consecutive token ranges, and
    // empty ones end where they start
    while (j0 >= e_end && e + 1 < p.n_entries) {
      ++e;
      enter();
    }
    const int nvalid = min(BN, total_tokens - j0);
    if (e_end - j0 >= BN) {
      const char* base = e_rows + (int64_t)(j0 - e_tok) * D * (int64_t)sizeof(bf16);
      const char* kt = base + g.k_off;
      const char* vt = base + g.v_off;
#pragma unroll
      for (int pp = 0; pp < PP; ++pp) {
        kreg[pp] = *reinterpret_cast<const bf16x8*>(kt + lane_off + pp * RPP * D * sizeof(bf16));
        vreg[pp] = *reinterpret_cast<const bf16x8*>(vt + lane_off + pp * RPP * D * sizeof(bf16));
      }
      return nvalid;
    }
    if (e_end - j0 + n_len >= nvalid) {
      // two pages: tile rows r < b1 are entry e's, the rest the next
      // entry's first rows; rows past the last token read row 0
      const int b1 = e_end - j0;
      const char* base_a = e_rows + (int64_t)(j0 - e_tok) * D * (int64_t)sizeof(bf16);
      const char* base_b = n_rows - (int64_t)b1 * D * (int64_t)sizeof(bf16);
#pragma unroll
      for (int pp = 0; pp < PP; ++pp) {
        const int r0 = lrow + RPP * pp;
        const int r = r0 < nvalid ? r0 : 0;
        const char* row = (r < b1 ? base_a : base_b) + (uint32_t)(r * D * sizeof(bf16) + lchunk * 8 * sizeof(bf16));
        kreg[pp] = *reinterpret_cast<const bf16x8*>(row + g.k_off);
        vreg[pp] = *reinterpret_cast<const bf16x8*>(row + g.v_off);
      }
      return nvalid;
    }
    int64_t off[PP];
    int es = e, seg_start = 0, page_row = j0 - tab[e].tok_start;
    for (int it = 0; it < BN; ++it) {  // each segment holds at least one row
      const int seg_end = min(nvalid, seg_start + tab[es].len - page_row);
      // row r of this segment is page row page_row + (r - seg_start)
      const int64_t base = (int64_t)tab[es].phys * g.page_bytes +
                           (head_off + (int64_t)(page_row - seg_start) * D) * (int64_t)sizeof(bf16);
#pragma unroll
      for (int pp = 0; pp < PP; ++pp) {
        const int r = lrow + RPP * pp;
        if (es == e || (r >= seg_start && r < seg_end))
          off[pp] = base + (int64_t)(r < nvalid ? r : seg_start) * (D * sizeof(bf16));
      }
      if (seg_end >= nvalid || es + 1 >= p.n_entries) break;
      seg_start = seg_end;
      page_row = 0;
      do {
        ++es;
      } while (tab[es].len == 0 && es + 1 < p.n_entries);  // the next entry with tokens
    }
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
      const char* row = p.pool + off[pp] + lchunk * 8 * sizeof(bf16);
      kreg[pp] = *reinterpret_cast<const bf16x8*>(row + g.k_off);
      vreg[pp] = *reinterpret_cast<const bf16x8*>(row + g.v_off);
    }
    return nvalid;
  };
  auto stage = [&](int b, int nvalid) {
    if (nvalid < BN) {
      // keys past the last token: zero V rows (their probabilities are 0)
#pragma unroll
      for (int pp = 0; pp < PP; ++pp)
        if (lrow + RPP * pp >= nvalid) vreg[pp] = bf16x8{};
    }
#pragma unroll
    for (int pp = 0; pp < PP; ++pp) {
      const int r = lrow + RPP * pp;
      *reinterpret_cast<bf16x8*>(&Ks[b][r * LDS_LD + lchunk * 8]) = kreg[pp];
      *reinterpret_cast<bf16x8*>(&Vs[b][r * LDS_LD + lchunk * 8]) = vreg[pp];
    }
  };

  const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
  const f32x16 zero = {};
  const int krow0 = perm_key(ql);
  // V^T operand of lane l for one MFMA step: keys 8*(l/32) + 0..7, column l%32.
  // Transposing-read addresses: lane L names key row 8*(L/32) + (L/4)%4 and
  // columns 16*((L/16)%2) + 4*(L%4) + 0..3; a second read 4 rows lower gives
  // keys 4..7.
  const int vtr_row = 8 * (lane >> 5) + ((lane >> 2) & 3);
  const int vtr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int nv_cur = BN, nv_nxt = BN;
  if (t_begin < t_end) {
    nv_cur = load_tile(t_begin);
    stage(0, nv_cur);
    if (t_begin + 1 < t_end) nv_nxt = load_tile(t_begin + 1);
  }

  for (int t = t_begin; t < t_end; ++t) {
    const int b = (t - t_begin) & 1;
    __syncthreads();  // tile t is in buffer b; buffer b^1 (tile t-1) is free
    const int nvalid = nv_cur;
    int nv_after = BN;

    // S^T = K_pi Q^T for both query blocks; each K operand feeds two MFMAs
    f32x16 sc[2][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[b][(32 * kb + krow0) * LDS_LD + ks * 16 + grp * 8]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ks], ks == 0 ? zero : sc[qb][kb], 0, 0, 0);
      }
    // Stage tile t+1 into the free buffer and start tile t+2's global loads
    // only now: every K-operand read of this tile has been issued and no V^T
    // read has, so the LDS writes drain during the softmax without queueing
    // ahead of either operand stream (6% faster than staging right after the
    // barrier; placements inside the QK products or after the softmax gain
    // nothing).  The next barrier orders the writes before their use.
    if (t + 1 < t_end) stage(b ^ 1, nv_nxt);
    if (t + 2 < t_end) nv_after = load_tile(t + 2);

    bf16x8 pb[2][2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // key of accumulator register r of block kb: 32*kb + 16*(r>>3) + 8*grp + (r&7)
      if (nvalid < BN) {
        // partial tile: keys at or past nvalid do not exist.  The empty asm
        // keeps the comparisons inside this branch (otherwise they are
        // speculated into every tile).
        int nv_lane = nvalid - 8 * grp;
        asm volatile("" : "+v"(nv_lane));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb + 16 * (r >> 3) + (r & 7) >= nv_lane) sc[qb][kb][r] = -INFINITY;
      }
      // Probabilities against the running max; the tile's row sum (v_dot2
      // over the bf16 probabilities) flags a tile whose largest probability
      // would pass 2^16 (or the first tile, where the max is still -inf and
      // the sum is inf or NaN).  Only then is the tile max taken, the max
      // raised, O and l rescaled and the tile redone.
      float nm = -m_run[qb];
      float lt = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pb[qb][kb][r >> 3][r & 7] = (bf16)__builtin_amdgcn_exp2f(fmaf(sc[qb][kb][r], p.scale_log2, nm));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bf16x2 pr = {pb[qb][kb][s][2 * j], pb[qb][kb][s][2 * j + 1]};
            lt = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lt, false);
          }
      if (__builtin_amdgcn_ballot_w64(!(lt <= 65536.f)) != 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[qb][kb][r]);
        mx = fmaxf(mx, wave_xor32(mx));
        const float m_new = fmaxf(m_run[qb], mx * p.scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) { oacc[qb][0][i] *= alpha; oacc[qb][1][i] *= alpha; }
        nm = -m_new;
        lt = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            pb[qb][kb][r >> 3][r & 7] = (bf16)__builtin_amdgcn_exp2f(fmaf(sc[qb][kb][r], p.scale_log2, nm));
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              bf16x2 pr = {pb[qb][kb][s][2 * j], pb[qb][kb][s][2 * j + 1]};
              lt = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lt, false);
            }
      }
      l_run[qb] += lt;
    }

    // O^T += V^T P^T for both query blocks; each V operand feeds two MFMAs
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const bf16* vp = &Vs[b][(32 * kb + 16 * s + vtr_row) * LDS_LD + 32 * db + vtr_col];
          const bf16x8 a = __builtin_shufflevector(lds_read_tr4(vp), lds_read_tr4(vp + 4 * LDS_LD), 0, 1, 2, 3, 4,
                                                   5, 6, 7);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb][kb][s], oacc[qb][db], 0, 0, 0);
        }
    nv_cur = nv_nxt;
    nv_nxt = nv_after;
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = l_run[qb] + wave_xor32(l_run[qb]);
    if (!qvalid[qb]) continue;
    if (p.splits == 1) {
      const float inv = 1.f / l_tot;
      bf16* out = static_cast<bf16*>(p.out) + ((int64_t)qrow[qb] * H + h) * D;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          bf16x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = (bf16)(oacc[qb][db][rb * 4 + j] * inv);
          *reinterpret_cast<bf16x4*>(out + 32 * db + 8 * rb + 4 * grp) = o;
        }
      if (p.lse && grp == 0) p.lse[(int64_t)qrow[qb] * H + h] = (m_run[qb] + __builtin_log2f(l_tot)) * kLn2;
    } else {
      const int64_t row = ((int64_t)sp * p.n_q + qrow[qb]) * H + h;
      float* po = p.part_o + row * D;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          f32x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = oacc[qb][db][rb * 4 + j];
          *reinterpret_cast<f32x4*>(po + 32 * db + 8 * rb + 4 * grp) = o;
        }
      if (grp == 0) {
        p.part_ml[row * 2 + 0] = m_run[qb];
        p.part_ml[row * 2 + 1] = l_tot;
      }
    }
  }
}

// Merge split-KV partials: O = sum_s 2^(m_s-m) O_s / sum_s 2^(m_s-m) l_s.
// Lanes take 4 consecutive d each (one 16-byte load per split and row).
//   G = 1 (up to 16 splits): 16 lanes per row, four rows per wave; lane j of
//     a row holds split j's m and weight, and sums all splits in order.
//   G = 4 (17 to 64 splits): one row per wave; lane l holds split l's m and
//     weight, and the four 16-lane groups sum every fourth split each before
//     their partial sums are added, which shortens each lane's dependent
//     chain fourfold for the many splits of a head-split layer.
// One wave per block, so that few rows still spread over every CU.
template <typename OutT, int G>
__global__ __launch_bounds__(64) void attend_combine_kernel(AttendParams p, int H) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  constexpr int W = 16 * G;  // lanes per row
  const int64_t rows = (int64_t)p.n_q * H;
  const int sub = threadIdx.x & 15;
  const int lr = threadIdx.x & (W - 1);  // lane within the row
  const int64_t idx = (int64_t)blockIdx.x * (4 / G) + threadIdx.x / W;
  if (idx >= rows) return;  // whole rows leave together
  const int S = p.splits;
  float ms = -INFINITY, ls = 0.f;
  if (lr < S) {
    ms = p.part_ml[((int64_t)lr * rows + idx) * 2];
    ls = p.part_ml[((int64_t)lr * rows + idx) * 2 + 1];
  }
  float m = ms;
#pragma unroll
  for (int off = W / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, W));
  const float w = lr < S ? __builtin_amdgcn_exp2f(ms - m) : 0.f;
  float L = w * ls;
#pragma unroll
  for (int off = W / 2; off >= 1; off >>= 1) L += __shfl_xor(L, off, W);
  f32x4v acc = {0.f, 0.f, 0.f, 0.f};
  const float* po = p.part_o + idx * D + 4 * sub;
  const int grp = lr >> 4;
#pragma unroll 8
  for (int s = grp; s < S; s += G) {
    const float ws = __shfl(w, s, W);
    const f32x4v o = *reinterpret_cast<const f32x4v*>(po + (int64_t)s * rows * D);
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = fmaf(ws, o[c], acc[c]);
  }
  if (G > 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc[c] += __shfl_xor(acc[c], 16, 64);
      acc[c] += __shfl_xor(acc[c], 32, 64);
    }
    if (grp != 0) return;
  }
  OutT* out = static_cast<OutT*>(p.out) + idx * D + 4 * sub;
#pragma unroll
  for (int c = 0; c < 4; ++c) out[c] = (OutT)(acc[c] / L);
  if (p.lse && lr == 0) p.lse[idx] = (m + __builtin_log2f(L)) * kLn2;
}

// fp32 caches: one wave per (query, head); lane = d.
__global__ __launch_bounds__(256) void attend_f32_kernel(PageGeom g, AttendParams p) {
  const int H = g.heads;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)p.n_q * H;
  if (wid >= rows) return;
  const int qrow = (int)(wid / H), h = (int)(wid % H);
  const float* q = static_cast<const float*>(p.q);
  const float qv = q[((int64_t)qrow * H + h) * D + lane];
  float m_run = -INFINITY, l_run = 0.f, o = 0.f;
  const DevEntry* tb = p.table + (int64_t)h * p.head_stride;
  for (int e = 0; e < p.n_entries; ++e) {
    const DevEntry en = tb[e];
    const char* page = p.pool + (int64_t)en.phys * g.page_bytes;
    const float* kt = reinterpret_cast<const float*>(page + g.k_off) + (int64_t)h * g.ts * D;
    const float* vt = reinterpret_cast<const float*>(page + g.v_off) + (int64_t)h * g.ts * D;
    for (int j = 0; j < en.len; ++j) {
      float s = qv * kt[(int64_t)j * D + lane];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
      const float x = s * p.scale_log2;
      const float m_new = fmaxf(m_run, x);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      const float pv = __builtin_amdgcn_exp2f(x - m_new);
      l_run = l_run * alpha + pv;
      o = o * alpha + pv * vt[(int64_t)j * D + lane];
      m_run = m_new;
    }
  }
  float* out = static_cast<float*>(p.out);
  out[((int64_t)qrow * H + h) * D + lane] = o / l_run;
  if (p.lse && lane == 0) p.lse[(int64_t)qrow * H + h] = (m_run + __builtin_log2f(l_run)) * kLn2;
}

}  // namespace

hipError_t attend_scratch_address(char** out) {
  static std::mutex mu;
  static char* addr[kAttendScratchDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kAttendScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<char*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_attend(const PageGeom& g, const AttendParams& p, bool bf16, hipStream_t s, hipEvent_t ev_start,
                         hipEvent_t ev_stop, const TableChunk* inl) {
  hipError_t err = ev_start ? hipEventRecord(ev_start, s) : hipSuccess;
  if (err != hipSuccess) return err;
  if (!bf16) {
    const int64_t rows = (int64_t)p.n_q * g.heads;
    attend_f32_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s>>>(g, p);
    err = hipGetLastError();
    return err == hipSuccess && ev_stop ? hipEventRecord(ev_stop, s) : err;
  }
  const int qtiles = (p.n_q + BM - 1) / BM;
  const int64_t nwg = (int64_t)qtiles * g.heads * p.splits;
  static const TableChunk kNoTable{};
  if (p.inline_table && (!inl || inl->count != p.n_entries || p.head_stride != 0)) return hipErrorInvalidValue;
  const TableChunk& tc = p.inline_table ? *inl : kNoTable;
  if (p.packed)
    attend_bf16_kernel<true><<<dim3((unsigned)nwg), dim3(256), 0, s>>>(g, p, qtiles, tc);
  else
    attend_bf16_kernel<false><<<dim3((unsigned)nwg), dim3(256), 0, s>>>(g, p, qtiles, tc);
  err = hipGetLastError();
  if (err == hipSuccess && ev_stop) err = hipEventRecord(ev_stop, s);
  if (err != hipSuccess || p.splits == 1) return err;
  const int64_t rows = (int64_t)p.n_q * g.heads;
  if (p.splits <= 16)
    attend_combine_kernel<__bf16, 1><<<dim3((unsigned)((rows + 3) / 4)), dim3(64), 0, s>>>(p, g.heads);
  else
    attend_combine_kernel<__bf16, 4><<<dim3((unsigned)rows), dim3(64), 0, s>>>(p, g.heads);
  return hipGetLastError();
}

}  // namespace kvs
