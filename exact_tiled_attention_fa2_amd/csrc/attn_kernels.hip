// Exact tiled attention forward for gfx950 (CDNA4): MFMA tile kernel with the
// RescaleThreshold + max-lagging online softmax, and the split-KV combine.
//
// Method: release page "v1.7 / flash_attn 2.9.2.post1", section 1.2 (skip the
// O/row_sum rescale while the row max rises by at most tau = 8 in log2 units,
// and keep the previous max on a skip so O, row_sum and P share one base);
// release page "FA2 2.9.0 Kernel Changes in v1.2", sections 1-3 (the rescale
// step, the exp2-domain probabilities with the -inf guard, the first KV step
// that never skips, and the split-KV variant of the row-block kernel).
//
// Layout of one workgroup (NW wave64s: 8 for large grids of D = 128 without
// softcap and of D = 256 without ALiBi, 4 otherwise, at two or three waves
// per SIMD; 32 query rows per wave):
//  * Each wave owns 32 query rows.  Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16: A = a 32-key slice of K read
//    from LDS, B = the wave's Q fragment held in VGPRs for the whole loop.
//    In the 32x32 accumulator a lane holds one query (lane % 32) and 16 keys
//    (8*(r/4) + 4*(lane/32) + r%4), so a row max is a register-local max
//    plus one exchange with lane ^ 32, and each lane keeps its own m and l.
//  * O^T = V^T P^T with the same MFMA.  The B operand (P^T, keys x queries)
//    is the converted score registers themselves: registers 0-7 of a 32-key
//    accumulator hold, per lane half, keys {0-3, 8-11} or {4-7, 12-15} of
//    a 16-key slice, so the contraction runs over the keys in that order.
//    The A operand (V^T) must use the same key order; it is read from the
//    row-major V tile in LDS with ds_read_b64_tr_b16, whose 16-lane
//    transpose hands lane l the element l % 4 of the rows addressed by
//    lanes 4j + l / 4 -- two such reads give the 8 keys of one lane.
//  * K and V tiles (BK keys x D) stream HBM -> LDS with 16-byte
//    buffer_load ... lds copies (no VGPR staging, one 32-bit offset register
//    per copy), double-buffered in LDS (one barrier per KV step); the copies
//    of step j+1 are in flight while step j computes.  16-byte chunks of a
//    row are XOR-swizzled so that both the K reads (8/16 rows, same chunk)
//    and the transposing V reads (4 rows x 2 chunks) hit distinct banks.
//  * Masks run only on KV steps that cross a mask edge for the wave; steps
//    that are fully masked for a wave are skipped by that wave.
//  * Keys at or beyond the valid length are never loaded (the last partial
//    step re-reads the last valid row and masks it), so NaN in unused cache
//    rows cannot reach the output.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

// Work item of one workgroup.  Work items are (query tile, head, batch x
// split).  Workgroups are dealt round-robin to the 8 XCDs (each with its own
// L2), so workgroup `lin` runs on XCD lin % 8 as that XCD's (lin / 8)-th
// workgroup.  The (head, batch x split) columns are dealt to the XCDs in
// turn, in chunks of p.xcd_chunk columns: single columns for varlen (every
// sequence spread over all XCDs keeps their loads even when lengths differ),
// one contiguous block per XCD otherwise (the heads of one key row stay on
// one XCD, which keeps DRAM pages together).  Each XCD walks its columns
// in groups of
// p.col_group columns whose K/V fit in its L2; inside a group it runs the
// heaviest query tile of every column first, so long causal tiles start early
// and short ones fill the tail (longest-first order).  Returns false when the
// tile holds no rows.
struct TileWork {
  int b, split, head, kvh;
  int q_start, k_start, sq, sk;
  int G, packed, m0, off;
  int blk_lo, blk_hi;  // this split's KV steps [blk_lo, blk_hi)
};

template <int BQ, int BK>
__device__ __forceinline__ bool tile_work(const FwdKernelParams& p, TileWork& w) {
  int mt, head, zz;
  {
    const int ny = gridDim.y;
    const int nmt = p.num_m_tiles;
    const int hz_total = ny * (int)gridDim.z;  // (head, batch x split) columns
    const int lin = (int)blockIdx.x + (int)gridDim.x * ((int)blockIdx.y + ny * (int)blockIdx.z);
    int col, rank;
    if ((hz_total & 7) == 0) {
      const int per_xcd = hz_total >> 3;
      const int k = lin >> 3;                       // position in this XCD's sequence
      const int cg = p.col_group;                   // columns per group
      const int grp = k / (cg * nmt);
      const int c0 = grp * cg;                      // first column of the group
      const int gcols = min(cg, per_xcd - c0);      // the last group may be narrower
      const int k2 = k - grp * cg * nmt;
      rank = k2 / gcols;
      const int lc = c0 + (k2 - rank * gcols);  // this XCD's column
      const int ch = p.xcd_chunk;
      col = ((lc / ch) * 8 + (lin & 7)) * ch + lc % ch;
    } else {
      rank = lin / hz_total;
      col = lin - rank * hz_total;
    }
    mt = nmt - 1 - rank;
    head = col % ny;  // q head, or kv head when packing
    zz = col / ny;
  }
  w.head = head;
  w.b = zz / p.num_splits;
  w.split = zz - w.b * p.num_splits;

  w.q_start = 0, w.k_start = 0, w.sq = p.seqlen_q, w.sk = p.seqlen_k;
  if (p.cu_seqlens_q != nullptr) {
    w.q_start = p.cu_seqlens_q[w.b];
    w.sq = p.cu_seqlens_q[w.b + 1] - w.q_start;
    w.k_start = p.cu_seqlens_k[w.b];
    w.sk = p.cu_seqlens_k[w.b + 1] - w.k_start;
  }
  if (p.seqused_k != nullptr) w.sk = min(max(p.seqused_k[w.b], 0), p.seqlen_k);
  w.G = p.pack_gqa ? p.group : 1;
  w.packed = w.sq * w.G;
  w.m0 = mt * BQ;
  if (w.m0 >= w.packed) return false;
  w.kvh = p.pack_gqa ? head : head / p.group;
  w.off = w.sk - w.sq;
  const int wl = p.window_left, wr = p.window_right;

  // KV range of the whole tile, then this split's share of whole KV steps.
  const int row_lo = w.m0 / w.G;
  const int row_hi = min(w.packed - 1, w.m0 + BQ - 1) / w.G;
  int n_lo = 0, n_hi = w.sk;
  if (wl >= 0) n_lo = max(0, row_lo + w.off - wl);
  if (wr >= 0) n_hi = min(w.sk, row_hi + w.off + wr + 1);
  int blk_lo = 0, blk_hi = 0;
  if (n_hi > n_lo) {
    blk_lo = n_lo / BK;
    blk_hi = (n_hi + BK - 1) / BK;
  }
  const int nblk = blk_hi - blk_lo;
  const int per = (nblk + p.num_splits - 1) / p.num_splits;
  const int s0 = blk_lo + w.split * per;
  w.blk_hi = min(blk_hi, s0 + per);
  w.blk_lo = s0;
  return true;
}

// Forward tile kernel.  NW waves per workgroup, each owning QG groups of 32
// query rows (BQ = 32 NW QG rows per workgroup); BK keys per KV step; LEAD
// LDS operand reads kept in flight ahead of the MFMAs; WPE waves per SIMD;
// NSTAGE K/V tile buffers (copies run NSTAGE - 1 steps ahead of compute);
// PAGED: K/V rows come from a paged cache through p.block_table.  ALIBI: the
// linear distance bias of p.alibi is added to the scores.
// 2^x without the transcendental unit (the exp2-on-FMA-pipe idea the pages
// name for FA4, release notes of the project survey page): Cody-Waite range
// reduction x = n + f with n = rint(x), |f| <= 1/2, a degree-4 polynomial for
// 2^f (coefficients fitted for least relative error on [-1/2, 1/2]: max
// relative error 2.6e-6, far below the 16-bit rounding of P), then 2^n by
// ldexp.  Inputs below -126, the -inf of a masked score included, give 0.
__device__ __forceinline__ float exp2_fma(float x) {
  const bool live = x >= -126.0f;
  const float xc = live ? x : 0.0f;
  const float n = __builtin_rintf(xc);
  const float f = xc - n;
  float p = 0.009571806527674198f;
  p = fmaf(p, f, 0.05591800436377525f);
  p = fmaf(p, f, 0.24024702608585358f);
  p = fmaf(p, f, 0.6931217908859253f);
  p = fmaf(p, f, 0.9999992847442627f);
  const float r = __builtin_amdgcn_ldexpf(p, (int)n);
  return live ? r : 0.0f;
}

template <class Ty, int D, int BK, int NW, int QG, bool SOFTCAP, int LEAD, int WPE, int NSTAGE = 2,
          bool PAGED = false, bool ALIBI = false, bool EXPP = false, int CPOL = 0, bool EPI_STAGE = true>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(WPE, WPE)))
fwd_tile_kernel(const FwdKernelParams p) {
  constexpr int NT = NW * 64;           // threads per workgroup
  constexpr int BQ = 32 * NW * QG;      // query rows (packed row/head pairs) per workgroup
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int ROWB = D * 2;           // bytes per LDS row
  constexpr int TILEB = BK * ROWB;      // bytes per K (or V) tile
  constexpr int KT = BK / 32;           // 32-key MFMA tiles per KV step
  constexpr int DS = D / 16;            // MFMA k-steps over the head dim (QK^T)
  constexpr int DT = D / 32;            // 32-wide head-dim tiles of O^T
  constexpr int KS = BK / 16;           // MFMA k-steps over keys (PV)
  constexpr int LOADS = BK * CH / NT;   // 16-byte copies per lane per tile
  constexpr int SWZ_MASK = CH < 16 ? CH - 1 : 15;
  static_assert(LOADS >= 1 && (BK * CH) % NT == 0, "tile must split evenly over the workgroup");

  // NSTAGE K and V tile buffers, as separate arrays so that each copy's
  // target is known at compile time (steps are unrolled by NSTAGE).
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "2 to 4 stages");
  __shared__ __attribute__((aligned(16))) char lds_k0[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_k1[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_k2[NSTAGE > 2 ? TILEB : 16];
  __shared__ __attribute__((aligned(16))) char lds_k3[NSTAGE > 3 ? TILEB : 16];
  __shared__ __attribute__((aligned(16))) char lds_v0[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_v1[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_v2[NSTAGE > 2 ? TILEB : 16];
  __shared__ __attribute__((aligned(16))) char lds_v3[NSTAGE > 3 ? TILEB : 16];
  auto kbuf = [&](auto st) __attribute__((always_inline)) -> char* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return lds_k0;
    else if constexpr (S == 1) return lds_k1;
    else if constexpr (S == 2) return lds_k2;
    else return lds_k3;
  };
  auto vbuf = [&](auto st) __attribute__((always_inline)) -> char* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return lds_v0;
    else if constexpr (S == 1) return lds_v1;
    else if constexpr (S == 2) return lds_v2;
    else return lds_v3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;  // which half of the wave: selects keys 4..7 of every 8

  TileWork w;
  if (!tile_work<BQ, BK>(p, w)) return;
  const int b = w.b, split = w.split, head = w.head, kvh = w.kvh;
  const int q_start = w.q_start, k_start = w.k_start, sq = w.sq, sk = w.sk;
  const int G = w.G, packed = w.packed, m0 = w.m0, off = w.off;
  const int blk_lo = w.blk_lo, blk_hi = w.blk_hi;
  const int wl = p.window_left, wr = p.window_right;
  (void)sq;
  (void)head;

  // ---------------------------------------------------------------- this lane's queries
  // Row blocks of 32 QG packed rows are dealt to the waves so that the two
  // waves sharing a SIMD (w and w + NW/2) hold an early and a late block:
  // blocks 0, 2, 4, .. go to the first half, .., 5, 3, 1 to the second.  On
  // causal diagonal tiles early blocks skip more fully masked steps, so this
  // evens out the work per SIMD.  Group g of the wave covers packed rows
  // [m0 + 32 (QG rb + g), +32).
  const int rb = wave < NW / 2 ? 2 * wave : NW - 1 - 2 * (wave - NW / 2);
  int row[QG], hq[QG], kmin[QG], kmax[QG], grow_lo[QG], grow_hi[QG];
  uint32_t kspan[QG];
  bool q_valid[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const int gpq_lo = m0 + 32 * (QG * rb + g);
    const int pq = gpq_lo + l32;
    q_valid[g] = pq < packed;
    row[g] = q_valid[g] ? pq / G : 0;
    hq[g] = p.pack_gqa ? head * G + (q_valid[g] ? pq - row[g] * G : 0) : head;
    grow_lo[g] = gpq_lo / G;
    grow_hi[g] = min(packed - 1, gpq_lo + 31) / G;
    // Key bounds visible to this lane's row (inclusive), including the valid
    // length; keys are never negative, so the lower bound is at least 0 and
    // both bounds and their difference stay within int range.
    kmin[g] = (wl >= 0) ? max(row[g] + off - wl, 0) : 0;
    kmax[g] = min(sk - 1, (wr >= 0) ? row[g] + off + wr : 0x3fffffff);
    kspan[g] = kmax[g] >= kmin[g] ? (uint32_t)(kmax[g] - kmin[g] + 1) : 0u;  // visible keys
  }
  // ALiBi slope of this lane's query head, in raw-score units.
  float slope[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g)
    slope[g] = ALIBI ? p.alibi[(int64_t)b * p.alibi_bstride + hq[g]] * p.alibi_inv_scale : 0.0f;

  // A wave whose rows all lie past the end (decode packs only G x Sq rows)
  // skips the compute and only takes part in the tile copies; so does a wave
  // on a KV step where none of its rows sees any key (the causal / window
  // edge): every score would be masked, so the step changes nothing.
  const bool wave_live = m0 + 32 * QG * rb < packed;
  const int wk_lo = (wl >= 0) ? grow_lo[0] + off - wl : -0x40000000;
  const int wk_hi = min(sk - 1, (wr >= 0) ? grow_hi[QG - 1] + off + wr : 0x3fffffff);
  auto wave_sees = [&](int blk) __attribute__((always_inline)) -> bool {
    const int j0 = blk * BK;
    return j0 <= wk_hi && j0 + BK - 1 >= wk_lo;
  };

  // Q fragments (B operand of S^T = K Q^T): 8 consecutive dims per k-step.
  u32x4 qf[QG][DS];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const uint16_t* qbase = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_batch +
                            (int64_t)(q_start + row[g]) * p.q_row + (int64_t)hq[g] * p.q_head;
#pragma unroll
    for (int t = 0; t < DS; ++t) {
      if (q_valid[g]) {
        qf[g][t] = *reinterpret_cast<const u32x4*>(qbase + 16 * t + 8 * hl);
      } else {
        qf[g][t] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  // The Q loads stay in flight while the first tile copies are issued; the
  // prologue's wait (all vector memory) retires both together.

  // Per-lane LDS byte offsets of the MFMA operands (constant over the loop).
  // The swizzle changes only the low 4 bits of a chunk index, so with more
  // than 16 chunks per row (D = 256) chunks 16.. repeat the offsets of 0..
  // plus 256 bytes: only the first 16 chunks' offsets are kept in registers.
  constexpr int KOFF = CH > 16 ? 8 : DS;  // distinct K offsets (k-steps cover 2 chunks)
  constexpr int VOFF = CH > 16 ? 4 : DT;  // distinct V offsets (4 chunks per 32 dims)
  int k_off[KOFF];
  {
    const int sw = chunk_swizzle(lane & 15) & SWZ_MASK;
#pragma unroll
    for (int t = 0; t < KOFF; ++t) k_off[t] = l32 * ROWB + (((2 * t + hl) ^ sw) << 4);
  }
  auto koff = [&](int t) __attribute__((always_inline)) { return k_off[t % KOFF] + (t / KOFF) * 256; };
  int v_off[2][VOFF];
  {
    const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2) {
      const int vrow = 4 * hl + 8 * r2 + ((lane & 15) >> 2);
      const int x = cl ^ (chunk_swizzle(vrow) & SWZ_MASK);
#pragma unroll
      for (int dt = 0; dt < VOFF; ++dt) v_off[r2][dt] = vrow * ROWB + (((4 * dt) ^ x) << 4) + ((lane & 1) << 3);
    }
  }

  // HBM -> LDS tile copies.  Copy i of wave w fills LDS bytes
  // [(NW i + w) * 1024, +1024) of the tile; the lane that lands on row r,
  // chunk position pos fetches the global chunk pos ^ swizzle(r), which
  // produces the swizzled layout the operand reads expect.
  // With a paged cache the batch term moves into the per-tile page lookup.
  constexpr bool paged = PAGED;
  const char* kbase = reinterpret_cast<const char*>(p.k) +
                      2 * ((paged ? 0 : (int64_t)b * p.k_batch + (int64_t)k_start * p.k_row) + (int64_t)kvh * p.k_head);
  const char* vbase = reinterpret_cast<const char*>(p.v) +
                      2 * ((paged ? 0 : (int64_t)b * p.v_batch + (int64_t)k_start * p.v_row) + (int64_t)kvh * p.v_head);
  const int64_t k_rowb = 2 * p.k_row, v_rowb = 2 * p.v_row;
  const int64_t k_pageb = 2 * p.k_batch, v_pageb = 2 * p.v_batch;
  int cp_row[LOADS], cp_col[LOADS];  // tile row and global byte column of each copy
  uint32_t off_k[LOADS], off_v[LOADS];  // byte offset of each copy from the tile's first row
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int u = (NW * i + wave) * 64 + lane;
    const int r = u / CH, pos = u % CH;
    cp_row[i] = r;
    cp_col[i] = (pos ^ (chunk_swizzle(r & 15) & SWZ_MASK)) << 4;
    // Row strides are below 2^24 elements, so (BK - 1) rows + a column stay below 2^31 bytes.
    off_k[i] = (uint32_t)(r * (int)(2 * p.k_row) + cp_col[i]);
    off_v[i] = (uint32_t)(r * (int)(2 * p.v_row) + cp_col[i]);
  }
  // Page holding KV step blk of a paged cache (clamped into the pool); a
  // tile never straddles pages (the page size is a multiple of 64).
  // The lookup is wave-uniform and the table read-only, so it goes through
  // the scalar cache: a scalar load is counted by lgkmcnt, and waiting for its
  // result never drains the HBM -> LDS copies of later steps (a vector load
  // issued after them would).
  typedef const __attribute__((address_space(4))) int* ConstIntPtr;
  const ConstIntPtr btab = (ConstIntPtr)(uintptr_t)p.block_table;
  auto page_of = [&](int blk) __attribute__((always_inline)) -> int {
    return min(max(btab[(int64_t)b * p.bt_stride + blk * BK / p.page_size], 0), p.num_pages - 1);
  };
  auto copy_tile = [&](const char* gbase, int64_t rowb, int64_t pageb, char* tile, int blk, int pg,
                       const uint32_t (&off)[LOADS]) __attribute__((always_inline)) {
    const int j0 = blk * BK;
    const char* tb;  // row j0 of this tile
    if constexpr (paged) {
      tb = gbase + (int64_t)pg * pageb + (int64_t)(j0 % p.page_size) * rowb;
    } else {
      tb = gbase + (int64_t)j0 * rowb;
    }
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(tb);
    if (j0 + BK <= sk) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) dma16_buf<CPOL>(rs, off[i], tile + (NW * i + wave) * 1024);
    } else {
      // Last, partial step: rows at or past the valid length re-read row
      // sk-1 instead.  Their scores are masked to -inf, so P = 0 multiplies
      // finite values, and memory past the valid length (which may hold NaN)
      // is never touched.
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int r = min(cp_row[i], sk - 1 - j0);
        dma16_buf<CPOL>(rs, (uint32_t)(r * (int)rowb + cp_col[i]), tile + (NW * i + wave) * 1024);
      }
    }
  };

  // Running state: one query per lane and group (both halves hold the same m).
  float m_run[QG], l_run[QG];  // l_run: this half's partial row sum
  f32x16 acc[QG][DT];
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[g][dt] = f32x16{};
  }

#ifdef ATTN_ROW_STATS
  // Per-row rescale counters (debug build): first max, skips, rescales, largest P.
  uint32_t st_first[QG], st_skip[QG], st_resc[QG];
  float st_pmax[QG];
#pragma unroll
  for (int g = 0; g < QG; ++g) st_first[g] = st_skip[g] = st_resc[g] = 0u, st_pmax[g] = 0.0f;
#endif

  const float c2 = p.scale_log2;
  const float tau = p.tau;
  // Rescale threshold in units of the raw score: the running max may lag the
  // block max by up to tau / c2 before O and l are rescaled.
  const float tau_raw = tau / c2;
  const int n = blk_hi - blk_lo;

  // ---- the three pieces of a KV step, on persistent per-wave registers
  f32x16 sc[QG][KT];      // scores of the step being processed
  uint32_t pk[QG][KT][8];  // its probabilities, packed to 16 bits

  // S^T = K Q^T: each K operand read feeds all QG groups.
  auto qk_part = [&](const char* k_cur) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < QG; ++g)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) sc[g][kt] = f32x16{};
#pragma unroll
    for (int t = 0; t < DS; ++t) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(k_cur + kt * 32 * ROWB + koff(t));
#pragma unroll
        for (int g = 0; g < QG; ++g) sc[g][kt] = Ty::mfma(a, qf[g][t], sc[g][kt]);
      }
    }
  };
  // Softcap, masks, RescaleThreshold with lagging, P = exp2(...), row sums, pack.
  auto softmax_part = [&](int blk) __attribute__((always_inline)) {
    const int j0 = blk * BK;
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      // ---- softcap, and masks where an edge crosses this step for the group
      if constexpr (SOFTCAP) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int r2 = 0; r2 < 16; ++r2)
            if constexpr (EXPP) {
              const float e = exp2_fma(sc[g][kt][r2] * p.softcap_pre * (2.0f * kLog2e));
              sc[g][kt][r2] = p.softcap * (1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f));
            } else {
              sc[g][kt][r2] = transform_score<SOFTCAP>(sc[g][kt][r2], p.softcap_pre, p.softcap);
            }
      }
      // ALiBi bias -slope |d| with d = i + off - key = d0 - c, where key =
      // j0 + 4 hl + c and c is fixed per register.  When the whole step lies
      // on one side of every row's diagonal, |d| is linear in c: the registers
      // take only +-slope c, and the lane constant -+slope d0 (kb) joins the
      // block max and the exponent's offset instead of every score.
      float kb = 0.0f;
      if constexpr (ALIBI) {
        const float d0 = (float)(row[g] + off - j0 - 4 * hl);
        if (grow_lo[g] + off >= j0 + BK - 1 || grow_hi[g] + off <= j0) {
          const float sl = (grow_lo[g] + off >= j0 + BK - 1) ? slope[g] : -slope[g];
          kb = -sl * d0;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r2 = 0; r2 < 16; ++r2)
              sc[g][kt][r2] = fmaf(sl, (float)(32 * kt + 8 * (r2 >> 2) + (r2 & 3)), sc[g][kt][r2]);
        } else {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r2 = 0; r2 < 16; ++r2) {
              const float c = (float)(32 * kt + 8 * (r2 >> 2) + (r2 & 3));
              sc[g][kt][r2] = fmaf(-slope[g], fabsf(d0 - c), sc[g][kt][r2]);
            }
        }
      }
      const int full_lo = (wl >= 0) ? grow_hi[g] + off - wl : -0x40000000;
      const int full_hi = min(sk - 1, (wr >= 0) ? grow_lo[g] + off + wr : 0x3fffffff);
      if (!(j0 >= full_lo && j0 + BK - 1 <= full_hi)) {
        // Visible iff key - kmin lies in [0, span) as one unsigned compare
        // (span = 0 for a row that sees no key; a key below kmin wraps to
        // at least 2^31 > span): one compare into VCC and one select per
        // score, where two compares into scalar register pairs ran the
        // kernel out of scalar registers.
        const uint32_t base = (uint32_t)(j0 + 4 * hl - kmin[g]);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
          for (int r2 = 0; r2 < 16; ++r2) {
            const uint32_t rel = base + (uint32_t)(32 * kt + 8 * (r2 >> 2) + (r2 & 3));
            sc[g][kt][r2] = rel < kspan[g] ? sc[g][kt][r2] : -INFINITY;
          }
        }
      }
      // ---- block max of this lane's keys (one half of the row)
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) mx = fmaxf(mx, sc[g][kt][r2]);
      if constexpr (ALIBI) mx += kb;
      // ---- RescaleThreshold with max lagging.  While no row's block max
      // rises more than tau above its running max, the running max is kept
      // (no exchange between the two halves is needed for that).  Otherwise
      // the halves agree on the row max and rows that rose too far rescale.
      [[maybe_unused]] const float m_before = m_run[g];
      if (__any(mx > m_run[g] + tau_raw)) {
        const float mx_row = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[g], mx_row);
        const float m_new_g = (m_new == -INFINITY) ? 0.0f : m_new;
        const float diff = (m_run[g] - m_new_g) * c2;  // <= 0; -inf on the first live step
        if (!(diff >= -tau)) {
          const float alpha = fast_exp2(diff);
          l_run[g] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[g][dt] *= alpha;
          m_run[g] = m_new;
        }
      }
#ifdef ATTN_ROW_STATS
      if (p.row_stats != nullptr) {  // wave-uniform
        const float mrow = fmaxf(mx, __shfl_xor(mx, 32));
        // A live row that rescales moves its running max up (the new max exceeds the old one by
        // more than the threshold); a skip leaves it in place.  Selects, not branches: divergent
        // branches here made the compiler move the accumulators to scratch memory.
        if (mrow > -INFINITY) {  // the row sees a key of this step
          const bool first = m_before == -INFINITY;
          st_first[g] += first ? 1u : 0u;
          st_resc[g] += (!first && m_run[g] != m_before) ? 1u : 0u;
          st_skip[g] += (!first && m_run[g] == m_before) ? 1u : 0u;
        }
      }
#endif
      // ---- P = exp2((s - m) c2) <= exp2(tau), row sum, 16-bit pack
      const float mg = (m_run[g] == -INFINITY) ? 0.0f : m_run[g];
      const float nb = ALIBI ? (kb - mg) * c2 : -mg * c2;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int r2 = 0; r2 < 16; r2 += 2) {
          const float p0 = EXPP ? exp2_fma(fmaf(sc[g][kt][r2], c2, nb)) : fast_exp2(fmaf(sc[g][kt][r2], c2, nb));
          const float p1 = EXPP ? exp2_fma(fmaf(sc[g][kt][r2 + 1], c2, nb))
                                : fast_exp2(fmaf(sc[g][kt][r2 + 1], c2, nb));
          l_run[g] += p0 + p1;
          pk[g][kt][r2 >> 1] = Ty::pack(p0, p1);
#ifdef ATTN_ROW_STATS
          st_pmax[g] = fmaxf(st_pmax[g], fmaxf(p0, p1));
#endif
        }
      }
    }
  };
  // O^T += V^T P^T: each V^T operand read feeds all QG groups.  Software-
  // pipelined by hand: the operand of the next MFMA is read before the current
  // one issues, so every MFMA finds its operand in flight one MFMA ahead (left
  // to the scheduler, the 256-register D = 256 tile read each operand right
  // before its MFMA and waited for it).  The softcap tiles keep the reads
  // grouped LEAD ahead by scheduling barriers (lead_pv), measured 1.7% faster
  // there; every other tile gained (D = 256 +5%, D = 128 +2%).
  auto pv_part = [&](const char* v_cur) __attribute__((always_inline)) {
    auto vread = [&](int idx) __attribute__((always_inline)) -> u32x4 {
      const int ks = idx / DT, dt = idx % DT;
      const int vo = ks * 16 * ROWB + (dt / VOFF) * 256;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v_cur + vo + v_off[0][dt % VOFF]));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(v_cur + vo + v_off[1][dt % VOFF]));
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
      const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
      return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
    };
    if constexpr (SOFTCAP) {
#pragma unroll
      for (int idx = 0; idx < KS * DT; ++idx) {
        const int ks = idx / DT, dt = idx % DT;
        const u32x4 aop = vread(idx);
#pragma unroll
        for (int g = 0; g < QG; ++g) {
          const u32x4 bop = {pk[g][ks >> 1][4 * (ks & 1) + 0], pk[g][ks >> 1][4 * (ks & 1) + 1],
                             pk[g][ks >> 1][4 * (ks & 1) + 2], pk[g][ks >> 1][4 * (ks & 1) + 3]};
          acc[g][dt] = Ty::mfma(aop, bop, acc[g][dt]);
        }
      }
      return;
    }
    u32x4 cur = vread(0);
#pragma unroll
    for (int idx = 0; idx < KS * DT; ++idx) {
      const int ks = idx / DT, dt = idx % DT;
      u32x4 nxt = cur;
      if (idx + 1 < KS * DT) nxt = vread(idx + 1);
#pragma unroll
      for (int g = 0; g < QG; ++g) {
        const u32x4 bop = {pk[g][ks >> 1][4 * (ks & 1) + 0], pk[g][ks >> 1][4 * (ks & 1) + 1],
                           pk[g][ks >> 1][4 * (ks & 1) + 2], pk[g][ks >> 1][4 * (ks & 1) + 3]};
        acc[g][dt] = Ty::mfma(cur, bop, acc[g][dt]);
      }
      cur = nxt;
    }
  };
  auto lead_pv = [&]() __attribute__((always_inline)) {
    if constexpr (LEAD > 0 && SOFTCAP) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * LEAD, 0);
      for (int i = 0; i < KS * DT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, QG, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  };
  auto lead_qk = [&]() __attribute__((always_inline)) {
    if constexpr (LEAD > 0) {  // keep LEAD operand reads in flight ahead of the MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, LEAD, 0);
      for (int i = 0; i < DS * KT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, QG, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
  };

  int pg_next = 0;  // page of the next in-loop copy (paged cache)

  // One KV step r with its tiles in stage ST = r % NSTAGE.  The copies for
  // step r + NSTAGE - 1 stream into the stage step r - 1 released.
  auto step = [&](auto st, int r) __attribute__((always_inline)) {
    constexpr int ST = decltype(st)::value;
    constexpr int FILL = (ST + NSTAGE - 1) % NSTAGE;
    const int blk = blk_lo + r;
    if (r + NSTAGE - 1 < n) {
      const int pg = pg_next;  // looked up one step ahead, off the copy's critical path
      if constexpr (paged) {
        if (r + NSTAGE < n) pg_next = page_of(blk + NSTAGE);
      }
      copy_tile(kbase, k_rowb, k_pageb, kbuf(std::integral_constant<int, FILL>{}), blk + NSTAGE - 1, pg, off_k);
      copy_tile(vbase, v_rowb, v_pageb, vbuf(std::integral_constant<int, FILL>{}), blk + NSTAGE - 1, pg, off_v);
    }
    if (wave_live && wave_sees(blk)) {  // otherwise the wave only helps with the copies
      qk_part(kbuf(std::integral_constant<int, ST>{}));
      lead_qk();
      softmax_part(blk);
      pv_part(vbuf(std::integral_constant<int, ST>{}));
      lead_pv();
    }
    // The copies for step r+1 must have landed; later steps' may still fly.
    // Copies are issued in step order, 2 LOADS per step per lane.
    const int later = min(NSTAGE - 2, n - 2 - r);  // steps r+2.. with copies in flight
    if constexpr (NSTAGE >= 4) {
      if (later >= 2) barrier_vmem_le<4 * LOADS>();
      else if (later == 1) barrier_vmem_le<2 * LOADS>();
      else barrier_vmem_le<0>();
    } else if constexpr (NSTAGE == 3) {
      if (later >= 1) barrier_vmem_le<2 * LOADS>();
      else barrier_vmem_le<0>();
    } else {
      barrier_vmem_le<0>();
    }
  };

  if (n > 0) {
    // Prologue: tiles of the first NSTAGE - 1 steps.
    {
      const int pg0 = paged ? page_of(blk_lo) : 0;
      copy_tile(kbase, k_rowb, k_pageb, lds_k0, blk_lo, pg0, off_k);
      copy_tile(vbase, v_rowb, v_pageb, lds_v0, blk_lo, pg0, off_v);
    }
    if constexpr (NSTAGE > 2) {
      if (n > 1) {
        const int pg1 = paged ? page_of(blk_lo + 1) : 0;
        copy_tile(kbase, k_rowb, k_pageb, lds_k1, blk_lo + 1, pg1, off_k);
        copy_tile(vbase, v_rowb, v_pageb, lds_v1, blk_lo + 1, pg1, off_v);
      }
    }
    if constexpr (NSTAGE > 3) {
      if (n > 2) {
        const int pg2 = paged ? page_of(blk_lo + 2) : 0;
        copy_tile(kbase, k_rowb, k_pageb, lds_k2, blk_lo + 2, pg2, off_k);
        copy_tile(vbase, v_rowb, v_pageb, lds_v2, blk_lo + 2, pg2, off_v);
      }
    }
    pg_next = (paged && NSTAGE - 1 < n) ? page_of(blk_lo + NSTAGE - 1) : 0;
    if constexpr (NSTAGE > 2) {
      // step 0's tiles must have landed; later prologue copies may still fly
      const int later = min(NSTAGE - 2, n - 1);
      if (NSTAGE >= 4 && later >= 2) barrier_vmem_le<4 * LOADS>();
      else if (later >= 1) barrier_vmem_le<2 * LOADS>();
      else barrier_vmem_le<0>();
    } else {
      barrier_vmem_le<0>();
    }
    int r = 0;
    for (; r + NSTAGE <= n; r += NSTAGE) {
      step(std::integral_constant<int, 0>{}, r);
      step(std::integral_constant<int, 1>{}, r + 1);
      if constexpr (NSTAGE > 2) step(std::integral_constant<int, 2>{}, r + 2);
      if constexpr (NSTAGE > 3) step(std::integral_constant<int, 3>{}, r + 3);
    }
    if (r < n) step(std::integral_constant<int, 0>{}, r);
    if (r + 1 < n) step(std::integral_constant<int, 1>{}, r + 1);
    if constexpr (NSTAGE > 2) {
      if (r + 2 < n) step(std::integral_constant<int, 2>{}, r + 2);
    }
  }

#ifdef ATTN_ROW_STATS
  if (p.row_stats != nullptr && p.o_part == nullptr) {  // one 16-byte record per valid row
#pragma unroll
    for (int g = 0; g < QG; ++g) {
      const float pm = fmaxf(st_pmax[g], __shfl_xor(st_pmax[g], 32));
      if (q_valid[g] && hl == 0) {
        const int64_t idx = (int64_t)b * p.lse_batch + (int64_t)hq[g] * p.lse_head + q_start + row[g];
        const u32x4 rec = {st_first[g], st_skip[g], st_resc[g], __builtin_bit_cast(uint32_t, pm)};
        *reinterpret_cast<u32x4*>(p.row_stats + 4 * idx) = rec;
      }
    }
  }
#endif

  // ---------------------------------------------------------------- epilogue
  // Staged store of O: a lane holds one query row, so direct 8-byte stores
  // scatter over 32 rows per instruction.  The wave instead writes its
  // 32 x D block into LDS (the K/V stage buffers are idle once the last
  // step's barrier has passed: every wave's reads of them have retired) and
  // reads it back row-contiguous, so that 64 / (D / 8) whole rows leave per
  // 16-byte-per-lane store.  Needs 16-byte aligned O rows.
  constexpr int REGB = 32 * ROWB;                        // one wave's 32-row block
  constexpr int RPBUF = TILEB / REGB;                    // blocks per stage buffer
  constexpr bool STAGED_O = EPI_STAGE && QG == 1 && RPBUF >= 1 && NW <= 2 * NSTAGE * RPBUF;
  if constexpr (STAGED_O) {
    const bool aligned = ((reinterpret_cast<uintptr_t>(p.o) & 15) | ((p.o_batch | p.o_row | p.o_head) & 7)) == 0;
    if (p.o_part == nullptr && aligned && n > 0) {
      char* reg;
      {
        const int bi = wave / RPBUF;                      // stage buffer: k0, k1, .., v0, v1, ..
        char* base;
        if (bi == 0) base = kbuf(std::integral_constant<int, 0>{});
        else if (bi == 1) base = kbuf(std::integral_constant<int, 1>{});
        else if (bi == NSTAGE) base = vbuf(std::integral_constant<int, 0>{});
        else base = vbuf(std::integral_constant<int, 1>{});
        if constexpr (NSTAGE > 2) {
          if (bi == 2) base = kbuf(std::integral_constant<int, 2>{});
          if (bi == NSTAGE + 2) base = vbuf(std::integral_constant<int, 2>{});
        }
        if constexpr (NSTAGE > 3) {
          if (bi == 3) base = kbuf(std::integral_constant<int, 3>{});
          if (bi == NSTAGE + 3) base = vbuf(std::integral_constant<int, 3>{});
        }
        reg = base + (wave % RPBUF) * REGB;
      }
      const float l_tot = l_run[0] + __shfl_xor(l_run[0], 32);
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      const float mgf = (m_run[0] == -INFINITY) ? 0.0f : m_run[0];
      const float lse_val = l_tot > 0.0f ? mgf * p.scale_ln + logf(l_tot) : -INFINITY;
      constexpr int SW = CH < 16 ? CH - 1 : 15;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int c = 4 * dt + g4;  // 16-byte chunk of dims 32 dt + 8 g4 .. + 7
          u32x2 w;
          w[0] = Ty::pack(acc[0][dt][4 * g4 + 0] * inv, acc[0][dt][4 * g4 + 1] * inv);
          w[1] = Ty::pack(acc[0][dt][4 * g4 + 2] * inv, acc[0][dt][4 * g4 + 3] * inv);
          *reinterpret_cast<u32x2*>(reg + l32 * ROWB + ((c ^ (l32 & SW)) << 4) + 8 * hl) = w;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes done
      asm volatile("" ::: "memory");
      constexpr int RPI = 64 / CH;  // rows per store instruction
#pragma unroll
      for (int it = 0; it < 32 / RPI; ++it) {
        const int rr = it * RPI + lane / CH;
        const int cc = lane % CH;
        const u32x4 v = *reinterpret_cast<const u32x4*>(reg + rr * ROWB + ((cc ^ (rr & SW)) << 4));
        const int rrow = __shfl(row[0], rr);
        const int rhq = __shfl(hq[0], rr);
        const int rvalid = __shfl((int)q_valid[0], rr);
        if (rvalid) {
          uint16_t* dst = reinterpret_cast<uint16_t*>(p.o) + (int64_t)b * p.o_batch +
                          (int64_t)(q_start + rrow) * p.o_row + (int64_t)rhq * p.o_head + 8 * cc;
          *reinterpret_cast<u32x4*>(dst) = v;
        }
      }
      if (q_valid[0] && hl == 0 && p.lse != nullptr)
        p.lse[(int64_t)b * p.lse_batch + (int64_t)hq[0] * p.lse_head + q_start + row[0]] = lse_val;
      return;
    }
  }
#pragma unroll
  for (int g = 0; g < QG; ++g) {
    const float l_tot = l_run[g] + __shfl_xor(l_run[g], 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const float mgf = (m_run[g] == -INFINITY) ? 0.0f : m_run[g];
    const float lse_val = l_tot > 0.0f ? mgf * p.scale_ln + logf(l_tot) : -INFINITY;
    if (!q_valid[g]) continue;
    if (p.o_part == nullptr) {
      uint16_t* op = reinterpret_cast<uint16_t*>(p.o) + (int64_t)b * p.o_batch +
                     (int64_t)(q_start + row[g]) * p.o_row + (int64_t)hq[g] * p.o_head;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * dt + 8 * g4 + 4 * hl;
          u32x2 w;
          w[0] = Ty::pack(acc[g][dt][4 * g4 + 0] * inv, acc[g][dt][4 * g4 + 1] * inv);
          w[1] = Ty::pack(acc[g][dt][4 * g4 + 2] * inv, acc[g][dt][4 * g4 + 3] * inv);
          *reinterpret_cast<u32x2*>(op + d0) = w;
        }
      }
      if (hl == 0 && p.lse != nullptr)
        p.lse[(int64_t)b * p.lse_batch + (int64_t)hq[g] * p.lse_head + q_start + row[g]] = lse_val;
    } else {
      const int64_t pr = (((int64_t)split * p.batch + b) * p.heads_q + hq[g]) * p.seqlen_q + row[g];
      float* op = p.o_part + pr * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * dt + 8 * g4 + 4 * hl;
          const f32x4 w = {acc[g][dt][4 * g4 + 0] * inv, acc[g][dt][4 * g4 + 1] * inv,
                           acc[g][dt][4 * g4 + 2] * inv, acc[g][dt][4 * g4 + 3] * inv};
          *reinterpret_cast<f32x4*>(op + d0) = w;
        }
      }
      if (hl == 0) p.lse_part[pr] = lse_val;
    }
  }
}

// Log-sum-exp merge of the split partials: LSE = M + ln sum_s exp(LSE_s - M),
// O = sum_s exp(LSE_s - LSE) O_s.  One wave per output row: lanes stride over
// the splits for the two reductions (fixed shuffle pattern), then every lane
// sums its D/64 dims over the splits in split order -- deterministic.  Empty
// splits carry LSE_s = -inf and weight 0.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <class Ty, int D>
__global__ void __launch_bounds__(256) combine_kernel(const CombineParams p) {
  constexpr int DPL = D / 64;  // dims per lane
  const int64_t rows = (int64_t)p.batch * p.heads_q * p.seqlen_q;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const int ns = p.num_splits;
  float mx = -INFINITY;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, p.lse_part[s * rows + r]);
  mx = wave_max(mx);
  float lse = -INFINITY;
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.0f;
  if (mx != -INFINITY) {
    float sum = 0.0f;
    for (int s = lane; s < ns; s += 64) sum += expf(p.lse_part[s * rows + r] - mx);
    sum = wave_sum(sum);
    lse = mx + logf(sum);
    const float* op = p.o_part + r * D + lane * DPL;
#pragma unroll 4
    for (int s = 0; s < ns; ++s) {
      const float ls = p.lse_part[s * rows + r];
      const float w = (ls == -INFINITY) ? 0.0f : expf(ls - lse);
      const float* src = op + s * rows * D;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[i] += w * src[i];
    }
  }
  const int row = (int)(r % p.seqlen_q);
  const int64_t bh = r / p.seqlen_q;
  const int hq = (int)(bh % p.heads_q);
  const int b = (int)(bh / p.heads_q);
  uint16_t* dst = reinterpret_cast<uint16_t*>(p.o) + (int64_t)b * p.o_batch + (int64_t)row * p.o_row +
                  (int64_t)hq * p.o_head + lane * DPL;
  if constexpr (DPL == 1) {
    f32x2 v2 = {o[0], 0.0f};
    *dst = (uint16_t)(Ty::pack(v2[0], v2[1]) & 0xffffu);
  } else {
#pragma unroll
    for (int i = 0; i < DPL; i += 2) *reinterpret_cast<uint32_t*>(dst + i) = Ty::pack(o[i], o[i + 1]);
  }
  if (lane == 0 && p.lse != nullptr) p.lse[r] = lse;
}

// Columns per longest-first group: as many as keep their K/V within an XCD's
// 4 MB L2, but at least two.  (With one column per group, all 32 CUs of an XCD
// read the same lines: at D = 256, where a column's K/V alone is 4 MB, that
// ran 1% slower than two columns, although it fetched 22% fewer HBM bytes.)
int col_group_for(const FwdKernelParams& p, int heads_grid, int nz, int head_dim) {
  const int64_t kv_bytes = 2 * (int64_t)std::max(p.seqlen_k, 1) * head_dim * 2 / p.num_splits;
  const int per_xcd = std::max(1, heads_grid * nz / 8);
  return (int)std::min<int64_t>(per_xcd, std::max<int64_t>(2, (int64_t(4) << 20) / kv_bytes));
}

template <class Ty, int D, int BK, int NW, int QG, bool SOFTCAP, int LEAD, int WPE, int NSTAGE = 2,
          bool PAGED = false, bool ALIBI = false, bool EXPP = false, int CPOL = 0, bool EPI_STAGE = true>
hipError_t launch_fwd_t(FwdKernelParams p, hipStream_t stream) {
  constexpr int BQ = 32 * NW * QG;
  const int64_t rows = (int64_t)p.seqlen_q * (p.pack_gqa ? p.group : 1);
  p.num_m_tiles = (int)((rows + BQ - 1) / BQ);
  const int heads_grid = p.pack_gqa ? p.heads_kv : p.heads_q;
  p.col_group = col_group_for(p, heads_grid, p.batch * p.num_splits, D);
  {
    // Varlen: single columns.  Otherwise one contiguous block per XCD
    // (measured best for equal-length columns: decode +1.6%, dense +1%).
    const int per_xcd = heads_grid * p.batch * p.num_splits / 8;
    p.xcd_chunk = (p.cu_seqlens_q == nullptr && per_xcd > 0) ? per_xcd : 1;
  }
  dim3 grid(p.num_m_tiles, heads_grid, p.batch * p.num_splits);
  note_block_k(BK);
  hipLaunchKernelGGL((fwd_tile_kernel<Ty, D, BK, NW, QG, SOFTCAP, LEAD, WPE, NSTAGE, PAGED, ALIBI, EXPP, CPOL, EPI_STAGE>), grid,
                     dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

// Tile-shape overrides of the debug build (set through attn_debug_set_variants;
// the release library compiles none of them): forward, D = 128: 1 = 128
// rows, 2 = 256 rows, 3 = 32-key steps with four stages, 4 = P (and
// softcap's tanh) with exp2 on the FMA pipe, 5 = 128 rows of 32-key steps at
// three waves per SIMD, 6 = 256 rows with O stored directly from the
// accumulator layout; D = 256: 1 = 128 rows, 2 = 256 rows, 3 = 128 rows at
// two waves per SIMD, 4 = 256 rows with the operand reads four ahead; D = 64:
// 1 = two waves per SIMD.  Decode: 1 = 32-key steps with four stages, 2 = K/V
// copies without the non-temporal policy.

template <class Ty, bool CAP, bool AL>
hipError_t launch_fwd_shape(const FwdKernelParams& p, int head_dim, hipStream_t stream) {
  // Decode-shaped launches (at most 64 live rows per tile after GQA packing)
  // read every K/V row exactly once: their copies carry the non-temporal
  // cache policy (CPOL_NT; streaming a 4 GiB cache this way ran 9% faster than
  // with the default policy).  Prefill tiles re-read each K/V tile from L2
  // (every query tile of a column needs it) and keep the default policy.
  const int64_t packed = (int64_t)p.seqlen_q * (p.pack_gqa ? p.group : 1);
  const bool stream_kv = packed <= 64 && !(kDebugBuild && dec_variant() == 2);
  if (p.block_table != nullptr) {  // paged cache: one tile shape per head dim
    switch (head_dim) {
      case 64:
        if (stream_kv) return launch_fwd_t<Ty, 64, 64, 4, 1, CAP, 4, 2, 2, true, AL, false, CPOL_NT>(p, stream);
        return launch_fwd_t<Ty, 64, 64, 4, 1, CAP, 4, 2, 2, true, AL>(p, stream);
      case 128:
        if (stream_kv) return launch_fwd_t<Ty, 128, 64, 4, 1, CAP, 4, 2, 2, true, AL, false, CPOL_NT>(p, stream);
        return launch_fwd_t<Ty, 128, 64, 4, 1, CAP, 4, 2, 2, true, AL>(p, stream);
      case 256:
        if (stream_kv) return launch_fwd_t<Ty, 256, 32, 4, 1, CAP, 4, 1, 2, true, AL, false, CPOL_NT>(p, stream);
        return launch_fwd_t<Ty, 256, 32, 4, 1, CAP, 4, 1, 2, true, AL>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (head_dim) {
    case 64: {
      // 128-row tiles at three waves per SIMD (129 registers at D = 64;
      // three workgroups per CU) except for decode-shaped launches and ALiBi;
      // variant 1 forces the two-wave tile.
      if constexpr (!AL) {
        if (packed > 64 && !(kDebugBuild && fwd_variant() == 1))
          return launch_fwd_t<Ty, 64, 64, 4, 1, CAP, 2, 3, 2>(p, stream);
      }
      if (stream_kv) return launch_fwd_t<Ty, 64, 64, 4, 1, CAP, 4, 2, 2, false, AL, false, CPOL_NT>(p, stream);
      return launch_fwd_t<Ty, 64, 64, 4, 1, CAP, 4, 2, 2, false, AL>(p, stream);
    }
    case 128: {
      if (packed <= 64) {
        // Decode-shaped launches (few live rows; the KV stream dominates).
        if constexpr (!AL && kDebugBuild) {
          // Variant 1: 32-key steps, four stages (three steps' copies in flight).
          if (dec_variant() == 1) return launch_fwd_t<Ty, 128, 32, 4, 1, CAP, 4, 2, 4, false, false, false, CPOL_NT>(p, stream);
        }
        if (stream_kv) return launch_fwd_t<Ty, 128, 64, 4, 1, CAP, 4, 2, 2, false, AL, false, CPOL_NT>(p, stream);
        return launch_fwd_t<Ty, 128, 64, 4, 1, CAP, 4, 2, 2, false, AL>(p, stream);
      }
      if constexpr (!AL && kDebugBuild) {  // tile overrides of the debug build
        switch (fwd_variant()) {
          case 1: return launch_fwd_t<Ty, 128, 64, 4, 1, CAP, 4, 2>(p, stream);
          case 2: return launch_fwd_t<Ty, 128, 64, 8, 1, CAP, 6, 2>(p, stream);
          case 3: return launch_fwd_t<Ty, 128, 32, 4, 1, CAP, 4, 2, 4>(p, stream);
          case 4:
            if (!CAP) return launch_fwd_t<Ty, 128, 64, 8, 1, CAP, 6, 2, 2, false, false, true>(p, stream);
            return launch_fwd_t<Ty, 128, 64, 4, 1, CAP, 4, 2, 2, false, false, true>(p, stream);
          case 5: return launch_fwd_t<Ty, 128, 32, 4, 1, CAP, 2, 3, 2>(p, stream);
          case 6: return launch_fwd_t<Ty, 128, 64, 8, 1, CAP, 6, 2, 2, false, false, false, 0, false>(p, stream);
          default: break;
        }
      }
      if constexpr (!AL) {
        // Softcap and varlen launches: 128-row tiles of 32-key steps at three
        // waves per SIMD (166 registers; three workgroups per CU, each SIMD
        // interleaving waves of three tiles) -- the VALU-heavier softcap step
        // and the uneven varlen tiles hide better behind the third wave.
        if (CAP || p.cu_seqlens_q != nullptr) return launch_fwd_t<Ty, 128, 32, 4, 1, CAP, 2, 3, 2>(p, stream);
      }
      // 256 query rows per workgroup (8 waves, one workgroup per CU) halve
      // the K/V re-reads from L2 per FLOP and win on dense and varlen
      // launches that give every CU at least two such workgroups; smaller
      // grids run faster with 128-row tiles (twice the workgroups), and so
      // does the VALU-heavy softcap path (two workgroups per CU).
      if (!CAP) {
        const int64_t heads_grid = p.pack_gqa ? p.heads_kv : p.heads_q;
        const int64_t wgs256 = (packed + 255) / 256 * heads_grid * p.batch * p.num_splits;
        if (wgs256 >= 2 * (int64_t)compute_units())
          return launch_fwd_t<Ty, 128, 64, 8, 1, CAP, 6, 2, 2, false, AL>(p, stream);
      }
      return launch_fwd_t<Ty, 128, 64, 4, 1, CAP, 4, 2, 2, false, AL>(p, stream);
    }
    case 256: {
      // 256 query rows at two waves per SIMD (8 waves of 256 registers: the
      // 32-key step keeps the O accumulators, Q fragments and scores within
      // 256) when the grid gives every CU two such workgroups; otherwise, for
      // decode-shaped launches and with ALiBi (whose slopes would spill), 128
      // rows at one wave per SIMD.  Variants 1 / 2 force 128 / 256 rows.
      if constexpr (!AL && kDebugBuild) {
        // 3: 128 rows at two waves per SIMD (two workgroups per CU); 4: 256 rows, operand lead 4.
        if (fwd_variant() == 3) return launch_fwd_t<Ty, 256, 32, 4, 1, CAP, 2, 2, 2, false, AL>(p, stream);
        if (fwd_variant() == 4) return launch_fwd_t<Ty, 256, 32, 8, 1, CAP, 4, 2, 2, false, AL>(p, stream);
      }
      if constexpr (!AL) {
        const int64_t heads_grid = p.pack_gqa ? p.heads_kv : p.heads_q;
        const int64_t wgs256 = (packed + 255) / 256 * heads_grid * p.batch * p.num_splits;
        const int v = kDebugBuild ? fwd_variant() : 0;
        if (v == 2 || (v != 1 && packed > 64 && wgs256 >= 2 * (int64_t)compute_units()))
          return launch_fwd_t<Ty, 256, 32, 8, 1, CAP, 2, 2, 2, false, AL>(p, stream);
      }
      if (stream_kv) return launch_fwd_t<Ty, 256, 32, 4, 1, CAP, 4, 1, 2, false, AL, false, CPOL_NT>(p, stream);
      return launch_fwd_t<Ty, 256, 32, 4, 1, CAP, 4, 1, 2, false, AL>(p, stream);
    }
    default:
      return hipErrorInvalidValue;
  }
}

template <class Ty, bool CAP>
hipError_t launch_fwd_cap(const FwdKernelParams& p, int head_dim, hipStream_t stream) {
  return p.alibi != nullptr ? launch_fwd_shape<Ty, CAP, true>(p, head_dim, stream)
                            : launch_fwd_shape<Ty, CAP, false>(p, head_dim, stream);
}

template <class Ty>
hipError_t launch_fwd_dtype(const FwdKernelParams& p, int head_dim, hipStream_t stream) {
  return p.softcap > 0.0f ? launch_fwd_cap<Ty, true>(p, head_dim, stream)
                          : launch_fwd_cap<Ty, false>(p, head_dim, stream);
}

template <class Ty, int D>
hipError_t launch_combine_t(const CombineParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.batch * p.heads_q * p.seqlen_q;
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL((combine_kernel<Ty, D>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <class Ty>
hipError_t launch_combine_dtype(const CombineParams& p, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_combine_t<Ty, 64>(p, stream);
    case 128: return launch_combine_t<Ty, 128>(p, stream);
    case 256: return launch_combine_t<Ty, 256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

#if !defined(ATTN_TU_DTYPE) || ATTN_TU_DTYPE == 0
hipError_t launch_fwd_f16(const FwdKernelParams& p, int head_dim, hipStream_t stream) {
  return launch_fwd_dtype<TypeF16>(p, head_dim, stream);
}
hipError_t launch_combine_f16(const CombineParams& p, int head_dim, hipStream_t stream) {
  return launch_combine_dtype<TypeF16>(p, head_dim, stream);
}
#endif
#if !defined(ATTN_TU_DTYPE) || ATTN_TU_DTYPE == 1
hipError_t launch_fwd_bf16(const FwdKernelParams& p, int head_dim, hipStream_t stream) {
  return launch_fwd_dtype<TypeBF16>(p, head_dim, stream);
}
hipError_t launch_combine_bf16(const CombineParams& p, int head_dim, hipStream_t stream) {
  return launch_combine_dtype<TypeBF16>(p, head_dim, stream);
}
#endif

}  // namespace attn
