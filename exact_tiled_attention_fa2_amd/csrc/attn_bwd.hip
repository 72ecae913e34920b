// Exact attention backward for gfx950 (CDNA4): dQ, dK, dV from the forward's
// saved LSE (the pages list the backward among the library's kernels and check
// its gradients against an fp32 reference: release page "v1.7 / flash_attn
// 2.9.2.post1", section 4.4; the forward's rescale threshold does not enter
// it, "FA2 2.9.0 Kernel Changes in v1.2", section 1).  For the loss whose
// gradient with respect to O is dO, with P recomputed from the scores and LSE:
//
//     dV = P^T dO,   dP = dO V^T,   dT = P (dP - D),   D_i = <dO_i, O_i>
//     dQ = scale * (dT g) K,   dK = scale * (dT g)^T Q
//
// where g = 1 - tanh^2 is the softcap derivative (1 without softcap) and
// D_i = sum_j P_ij dP_ij = <dO_i, O_i> is the softmax Jacobian's row term.
//
// Two kernels, in stream order, no atomics (every output element has one
// owner, so the result is deterministic):
//  * bwd_dq_kernel: one workgroup per 128- or 256-query tile of one query
//    head, the forward's orientation (a lane holds one query): S^T = K Q^T
//    and dP^T = V dO^T (A = K / V rows from LDS, B = Q / dO held in VGPRs),
//    the elementwise dS^T, then dQ^T += K^T dS^T (A = K^T read transposed
//    from the K tile).  It recomputes S and dP, which the dK/dV kernel also
//    forms: seven tile products instead of five, traded for no atomics.  It
//    also forms D = rowsum(dO * O) in fp32 for its queries (from the dO rows
//    it holds) and writes it for the next kernel.
//  * bwd_dkdv_pair_kernel: one workgroup per 128-key tile of one KV head.
//    32 keys belong to a pair of waves on one SIMD that walks the query tiles
//    of every query head of its GQA group: S = Q K^T and dP = dO V^T (A = Q /
//    dO rows read from LDS, B = the keys' K / V rows held in VGPRs), the
//    elementwise P and dS, then dV^T += dO^T P and dK^T += Q^T dS (A = Q^T /
//    dO^T read transposed from the same LDS tiles with ds_read_b64_tr_b16,
//    B = the packed P / dS registers); one wave of the pair forms S, P and
//    dV, the other dP, dS and dK.  In these accumulators a lane holds one key.
// Q/dO (dK/dV kernels, three stages) and K/V (dQ kernel, two stages) tiles
// stream HBM -> LDS with global_load_lds in the forward's XOR-swizzled layout.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

// One packed 16-bit pair -> two fp32 (exact).
template <class Ty>
__device__ __forceinline__ f32x2 unpack2(uint32_t u) {
  if constexpr (std::is_same<Ty, TypeBF16>::value) {
    return f32x2{__builtin_bit_cast(float, u << 16), __builtin_bit_cast(float, u & 0xffff0000u)};
  } else {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, u), f32x2);
  }
}

struct SeqRange {
  int q_start, k_start, sq, sk;
};

__device__ __forceinline__ SeqRange seq_range(const BwdKernelParams& p, int b) {
  SeqRange r{0, 0, p.seqlen_q, p.seqlen_k};
  if (p.cu_seqlens_q != nullptr) {
    r.q_start = p.cu_seqlens_q[b];
    r.sq = p.cu_seqlens_q[b + 1] - r.q_start;
    r.k_start = p.cu_seqlens_k[b];
    r.sk = p.cu_seqlens_k[b + 1] - r.k_start;
  }
  return r;
}

// LSE in exp2 units, with a row that saw no key (LSE = -inf) mapped to +inf
// so that every recomputed P of that row is exp2(-inf) = 0.
__device__ __forceinline__ float lse_to_exp2(float l) { return l == -INFINITY ? INFINITY : l * kLog2e; }

// Work item of a backward workgroup from its linear index.  The grid is
// (tiles, heads, batch); items are dealt tile-rank-major -- every (head,
// batch) column's rank-0 tile first, then rank 1, .. -- so the dispatcher
// starts the heaviest causal tiles first and fills the tail with light ones
// (in grid order the first wave of workgroups mixes all sizes and the
// makespan grows by ~30% on a causal square).  Workgroup i runs on XCD i % 8,
// so when the column count is a multiple of 8 all tiles of a column share
// one XCD and its L2.
struct TileRank {
  int rank, head, b;
};
__device__ __forceinline__ TileRank tile_rank() {
  const int cols = (int)gridDim.y * (int)gridDim.z;
  const int lin = (int)blockIdx.x + (int)gridDim.x * ((int)blockIdx.y + (int)gridDim.y * (int)blockIdx.z);
  const int c = lin % cols;
  return TileRank{lin / cols, c % (int)gridDim.y, c / (int)gridDim.y};
}

// HBM -> LDS copy of a tile of NR rows (one 16-byte chunk per lane per copy)
// in the forward's swizzled layout; rows at or past `valid` re-read row
// valid - 1 (their results are masked).
template <int NR, int D, int NT>
struct TileCopier {
  static constexpr int CH = D / 8;
  static constexpr int ROWB = D * 2;
  static constexpr int LOADS = NR * CH / NT;
  static constexpr int SWZ_MASK = CH < 16 ? CH - 1 : 15;
  static_assert(LOADS >= 1 && (NR * CH) % NT == 0, "tile must split evenly over the workgroup");
  int row[LOADS], col[LOADS];
  __device__ __forceinline__ void init(int wave, int lane, int nw) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int u = (nw * i + wave) * 64 + lane;
      const int r = u / CH, pos = u % CH;
      row[i] = r;
      col[i] = (pos ^ (chunk_swizzle(r & 15) & SWZ_MASK)) << 4;
    }
  }
  // tb: byte address of tile row 0; rowb: bytes between rows; valid: rows that exist.
  __device__ __forceinline__ void copy(const char* tb, int64_t rowb, int valid, char* tile, int wave,
                                       int nw) const {
    if (valid >= NR) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i)
        dma16(tb + (uint32_t)(row[i] * (int)rowb + col[i]), tile + (nw * i + wave) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int r = min(row[i], valid - 1);
        dma16(tb + (int64_t)r * rowb + col[i], tile + (nw * i + wave) * 1024);
      }
    }
  }
};

// Per-lane LDS byte offsets of the MFMA operands in the swizzled layout:
// row reads (A operand of a 32-row slice, 8 consecutive dims per lane) and
// transposing reads (A operand that contracts over 16 rows).  The swizzle
// changes only the low 4 bits of a chunk index, so with more than 16 chunks
// per row (D = 256) chunks 16.. sit at the offsets of chunks 0.. plus 256
// bytes: only the first 16 chunks' offsets are kept in registers (the rest
// become immediate offsets of the reads).
template <int D>
struct OperandOffsets {
  static constexpr int CH = D / 8;
  static constexpr int ROWB = D * 2;
  static constexpr int DS = D / 16;
  static constexpr int DT = D / 32;
  static constexpr int SWZ_MASK = CH < 16 ? CH - 1 : 15;
  static constexpr int NRO = CH > 16 ? 8 : DS;  // distinct row-read offsets (a k-step covers 2 chunks)
  static constexpr int NTO = CH > 16 ? 4 : DT;  // distinct transposing-read offsets (4 chunks per 32 dims)
  int row_off_[NRO];
  int tr_off_[2][NTO];
  __device__ __forceinline__ void init(int lane) {
    const int l32 = lane & 31, hl = lane >> 5;
    const int sw = chunk_swizzle(lane & 15) & SWZ_MASK;
#pragma unroll
    for (int t = 0; t < NRO; ++t) row_off_[t] = l32 * ROWB + (((2 * t + hl) ^ sw) << 4);
    const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2) {
      const int vrow = 4 * hl + 8 * r2 + ((lane & 15) >> 2);
      const int x = cl ^ (chunk_swizzle(vrow) & SWZ_MASK);
#pragma unroll
      for (int dt = 0; dt < NTO; ++dt) tr_off_[r2][dt] = vrow * ROWB + (((4 * dt) ^ x) << 4) + ((lane & 1) << 3);
    }
  }
  __device__ __forceinline__ int row_off(int t) const { return row_off_[t % NRO] + (t / NRO) * 256; }
  __device__ __forceinline__ int tr_off(int r2, int dt) const { return tr_off_[r2][dt % NTO] + (dt / NTO) * 256; }
};

// A operand for the contraction over the 16 rows of slice ks of a tile,
// 32 dims of block dt: two transposing reads.
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const char* tile, const OperandOffsets<D>& o, int ks, int dt) {
  constexpr int ROWB = D * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + ks * 16 * ROWB + o.tr_off(0, dt)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + ks * 16 * ROWB + o.tr_off(1, dt)));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
  const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
}

// Store a [D x 32] accumulator (lane = row of the output, registers = dims
// 32 dt + 8 (r / 4) + 4 (lane / 32) + r % 4) times `mul` as 16-bit.
template <class Ty, int D>
__device__ __forceinline__ void store_rows(uint16_t* dst, const f32x16 (&acc)[D / 32], float mul, int hl) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * dt + 8 * g4 + 4 * hl;
      u32x2 w;
      w[0] = Ty::pack(acc[dt][4 * g4 + 0] * mul, acc[dt][4 * g4 + 1] * mul);
      w[1] = Ty::pack(acc[dt][4 * g4 + 2] * mul, acc[dt][4 * g4 + 3] * mul);
      *reinterpret_cast<u32x2*>(dst + d0) = w;
    }
  }
}

// The same [D x 32] accumulator stored through LDS: the wave writes its
// 32 x D block into `region` (32 * 2D bytes, private to the wave and idle;
// 16-byte chunks XOR-swizzled by row) and reads it back row-contiguous, so
// that each 16-byte-per-lane store covers 64 / (D / 8) whole rows instead of
// scattering 8-byte pieces over 32 rows.  row_ptr(r) gives the destination
// of row r, or nullptr for a row that is not stored.
template <class Ty, int D, class RowPtr>
__device__ __forceinline__ void store_rows_staged(char* region, const f32x16 (&acc)[D / 32], float mul, int lane,
                                                  RowPtr row_ptr) {
  constexpr int CH = D / 8;
  constexpr int ROWB = 2 * D;
  constexpr int SW = CH < 16 ? CH - 1 : 15;
  constexpr int RPI = 64 / CH;  // rows per store instruction
  const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int c = 4 * dt + g4;
      u32x2 w;
      w[0] = Ty::pack(acc[dt][4 * g4 + 0] * mul, acc[dt][4 * g4 + 1] * mul);
      w[1] = Ty::pack(acc[dt][4 * g4 + 2] * mul, acc[dt][4 * g4 + 3] * mul);
      *reinterpret_cast<u32x2*>(region + l32 * ROWB + ((c ^ (l32 & SW)) << 4) + 8 * hl) = w;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes done
  asm volatile("" ::: "memory");
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int rr = it * RPI + lane / CH;
    const int cc = lane % CH;
    const u32x4 v = *reinterpret_cast<const u32x4*>(region + rr * ROWB + ((cc ^ (rr & SW)) << 4));
    uint16_t* d = row_ptr(rr);
    if (d != nullptr) *reinterpret_cast<u32x4*>(d + 8 * cc) = v;
  }
}

// 16-byte aligned rows (base pointer and every stride a multiple of 8 elements).
__device__ __forceinline__ bool rows_aligned16(const void* base, int64_t s0, int64_t s1, int64_t s2) {
  return ((reinterpret_cast<uintptr_t>(base) & 15) | ((s0 | s1 | s2) & 7)) == 0;
}

// ---------------------------------------------------------------- dK, dV
// NW waves per workgroup (32 keys each), WPE waves per SIMD.  PASSES = 1:
// one walk over the queries accumulates dV and dK together (~440 registers:
// one wave per SIMD).  PASSES = 2: a first walk accumulates dV (S, P), a
// second dK (S, dP, dS) -- S is formed twice, but each walk fits two waves
// per SIMD.
template <class Ty, int D, bool SOFTCAP, bool ALIBI, int NW, int WPE, int PASSES>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(WPE, WPE)))
bwd_dkdv_kernel(const BwdKernelParams p) {
  static_assert(PASSES == 1 || PASSES == 2, "one or two passes");
  constexpr int NT = NW * 64;
  // Queries per step: 64, or 32 at D = 256 (six stage tiles of 64 rows of
  // 512 bytes would not fit the 160 KB of LDS).
  constexpr int BQ = D > 128 ? 32 : 64;
  constexpr int QB = BQ / 32;       // 32-query MFMA blocks per step
  constexpr int BN = 32 * NW;       // keys per workgroup
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BQ * ROWB;
  constexpr int DS = D / 16;
  constexpr int DT = D / 32;
  using Copier = TileCopier<BQ, D, NT>;

  // Three stages of Q and dO tiles (copies run two steps ahead of compute);
  // the LSE / D rows of a step are staged one step ahead.
  __shared__ __attribute__((aligned(16))) char lds_q0[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_q1[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_q2[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_g0[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_g1[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_g2[TILEB];
  __shared__ __attribute__((aligned(16))) float lds_lse[2][BQ];
  __shared__ __attribute__((aligned(16))) float lds_dd[2][BQ];
  auto qbuf = [&](auto st) __attribute__((always_inline)) -> char* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return lds_q0;
    else if constexpr (S == 1) return lds_q1;
    else return lds_q2;
  };
  auto gbuf = [&](auto st) __attribute__((always_inline)) -> char* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return lds_g0;
    else if constexpr (S == 1) return lds_g1;
    else return lds_g2;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  const TileRank tr = tile_rank();  // rank = key tile: the first tiles see the most queries
  const int kvh = tr.head, b = tr.b;
  const SeqRange sr = seq_range(p, b);
  const int sq = sr.sq, sk = sr.sk, off = sk - sq;
  const int n0 = tr.rank * BN;
  if (n0 >= sk) return;
  const int wl = p.window_left, wr = p.window_right;
  const int G = p.group;

  // This lane's key and the wave's key range.
  const int wk_lo = n0 + 32 * wave;
  const int key = wk_lo + l32;
  const bool key_valid = key < sk;
  const int keyc = key_valid ? key : sk - 1;
  const bool wave_live = wk_lo < sk;
  const int wk_hi = min(sk - 1, wk_lo + 31);

  const uint16_t* kp = reinterpret_cast<const uint16_t*>(p.k) + b * p.k_batch +
                       (int64_t)(sr.k_start + keyc) * p.k_row + kvh * p.k_head;
  const uint16_t* vp = reinterpret_cast<const uint16_t*>(p.v) + b * p.v_batch +
                       (int64_t)(sr.k_start + keyc) * p.v_row + kvh * p.v_head;

  // Queries that see some key of this workgroup.
  const int wg_hi = min(sk - 1, n0 + BN - 1);
  const int q_lo = (wr >= 0) ? max(0, n0 - off - wr) : 0;
  const int q_hi = (wl >= 0) ? min(sq - 1, wg_hi - off + wl) : sq - 1;
  const int qblk_lo = q_lo / BQ;
  const int nsph = (q_hi >= q_lo) ? (q_hi / BQ + 1 - qblk_lo) : 0;  // steps per query head
  const int n = G * nsph;

  OperandOffsets<D> oo;
  oo.init(lane);
  Copier cp;
  cp.init(wave, lane, NW);

  const float c2 = p.scale_log2;
  const float icap = p.inv_softcap;

  // Steps walk the query tiles of each query head of the group in turn; a
  // step's (head, first query) advances by one tile, wrapping to the next head.
  auto advance = [&](int& h, int& q0) __attribute__((always_inline)) {
    q0 += BQ;
    if (q0 >= (qblk_lo + nsph) * BQ) {
      q0 = qblk_lo * BQ;
      ++h;
    }
  };
  // Tile copies of step (h, q0) into stage buffers qt / gt (2 LOADS per lane).
  auto issue = [&](int h, int q0, char* qt, char* gt) __attribute__((always_inline)) {
    const char* qb = reinterpret_cast<const char*>(p.q) +
                     2 * (b * p.q_batch + (int64_t)(sr.q_start + q0) * p.q_row + h * p.q_head);
    const char* gb = reinterpret_cast<const char*>(p.dout) +
                     2 * (b * p.do_batch + (int64_t)(sr.q_start + q0) * p.do_row + h * p.do_head);
    cp.copy(qb, 2 * p.q_row, sq - q0, qt, wave, NW);
    cp.copy(gb, 2 * p.do_row, sq - q0, gt, wave, NW);
  };
  // The (guarded) LSE / D loads of step r's queries, kept in registers until
  // they are staged to LDS at the end of the previous step.
  float st_lse = 0.0f, st_dd = 0.0f;
  auto issue_rows = [&](int h, int q0) __attribute__((always_inline)) {
    if (tid < BQ) {
      const int q = q0 + tid;
      const int64_t li = b * p.lse_batch + (int64_t)h * p.lse_head + sr.q_start + q;
      st_lse = q < sq ? p.lse[li] : -INFINITY;
      st_dd = q < sq ? p.dsum[li] : 0.0f;
    }
  };
  auto stage_rows = [&](int st) __attribute__((always_inline)) {
    if (tid < BQ) {
      lds_lse[st][tid] = lse_to_exp2(st_lse);
      lds_dd[st][tid] = st_dd;
    }
  };

  // One walk over the steps; DO_DV / DO_DK select the gradients it forms.
  auto run_pass = [&](auto pass_c) __attribute__((always_inline)) {
  constexpr int PASS = decltype(pass_c)::value;
  constexpr bool DO_DV = PASSES == 1 || PASS == 0;
  constexpr bool DO_DK = PASSES == 1 || PASS == 1;
  // K (and, for dK, V) rows of this lane's key: B operands (8 consecutive
  // dims per k-step), loaded per walk.
  u32x4 kf[DS], vf[DS];
#pragma unroll
  for (int t = 0; t < DS; ++t) {
    kf[t] = *reinterpret_cast<const u32x4*>(kp + 16 * t + 8 * hl);
    if constexpr (DO_DK) vf[t] = *reinterpret_cast<const u32x4*>(vp + 16 * t + 8 * hl);
  }
  f32x16 acc_dk[DT], acc_dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    acc_dk[dt] = f32x16{};
    acc_dv[dt] = f32x16{};
  }
  // Step r computes on stage ST = r % 3.  Its row loads (for r + 1) are
  // issued before its copies (for r + 2), so waiting until only the newest
  // 2 LOADS copies are outstanding retires everything step r + 1 needs.
  int h = kvh * G, q0 = qblk_lo * BQ;  // position of the step being computed
  auto step = [&](auto stc, int r) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
    constexpr int FILL = (ST + 2) % 3;
    char* q_cur = qbuf(stc);
    char* g_cur = gbuf(stc);
    int h1 = h, q1 = q0;
    advance(h1, q1);
    int h2 = h1, q2 = q1;
    advance(h2, q2);
    if (r + 1 < n) issue_rows(h1, q1);
    if (r + 2 < n) issue(h2, q2, qbuf(std::integral_constant<int, FILL>{}), gbuf(std::integral_constant<int, FILL>{}));
    const int qv_hi = min(sq - 1, q0 + BQ - 1);
    const bool sees = wave_live && (wr < 0 || wk_lo <= qv_hi + off + wr) && (wl < 0 || wk_hi >= q0 + off - wl);
    if (sees) {
      float slope = 0.0f;
      if constexpr (ALIBI) slope = p.alibi[b * p.alibi_bstride + h] * p.alibi_inv_scale;
      // Every (query, key) pair of the step and wave visible: no mask work.
      const bool full = q0 + BQ - 1 < sq && wk_lo + 31 < sk && (wr < 0 || wk_lo + 31 <= q0 + off + wr) &&
                        (wl < 0 || wk_lo >= q0 + BQ - 1 + off - wl);
      // The step's 32-query blocks one after the other (fewer live registers).
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        // One wave per SIMD hides no LDS latency behind another wave: all of
        // the block's operand reads are issued before its MFMAs.
        // In batches of RB k-steps (all of them at one wave per SIMD).
        // At D = 256 the K and V rows alone take 128 registers: batches of four.
        constexpr int RB = (WPE == 1 && D <= 128) ? DS : (D > 128 ? 4 : (DS >= 4 ? 2 : DS));
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int t0 = 0; t0 < DS; t0 += RB) {
          u32x4 aq[RB], ag[RB];
#pragma unroll
          for (int t = 0; t < RB; ++t) {
            aq[t] = *reinterpret_cast<const u32x4*>(q_cur + qb * 32 * ROWB + oo.row_off(t0 + t));
            if constexpr (DO_DK) ag[t] = *reinterpret_cast<const u32x4*>(g_cur + qb * 32 * ROWB + oo.row_off(t0 + t));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int t = 0; t < RB; ++t) {
            s = Ty::mfma(aq[t], kf[t0 + t], s);
            if constexpr (DO_DK) dp = Ty::mfma(ag[t], vf[t0 + t], dp);
          }
        }
        // At one wave per SIMD the transposed operands of the block's two
        // 16-query slices are read under the S / dP MFMAs (two reads after
        // each MFMA: a wave keeps at most 15 LDS reads in flight, so issued
        // in one batch they would stall it), ahead of the elementwise work;
        // at two waves per SIMD the other wave covers their latency and the
        // registers are needed elsewhere.
        constexpr bool TR_AHEAD = WPE == 1 && D <= 128;
        u32x4 tg[2][DT], tq[2][DT];
        if constexpr (TR_AHEAD) {
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              if constexpr (DO_DV) tg[k2][dt] = tr_operand<D>(g_cur, oo, 2 * qb + k2, dt);
              if constexpr (DO_DK) tq[k2][dt] = tr_operand<D>(q_cur, oo, 2 * qb + k2, dt);
            }
          }
          if constexpr (RB == DS) {
            constexpr int NM = DS * (DO_DK ? 2 : 1);                          // S (and dP) MFMAs
            constexpr int NR = 4 * DT * ((DO_DV ? 1 : 0) + (DO_DK ? 1 : 0));  // transposing reads
            static_assert(NR % NM == 0, "reads spread evenly over the MFMAs");
#pragma unroll
            for (int i = 0; i < NM; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, NR / NM, 0);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // P and dS, with the mask only on steps that an edge crosses for the
        // wave (two copies of the loop, so that full steps carry no mask work).
        uint32_t pp[8], ps[8];
        auto elementwise = [&](auto masked_c) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_c)::value;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int qo = 32 * qb + 8 * g4 + 4 * hl;  // first of this lane's 4 consecutive queries
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lds_lse[r & 1][qo]);
          f32x4 d4 = f32x4{};
          if constexpr (DO_DK) d4 = *reinterpret_cast<const f32x4*>(&lds_dd[r & 1][qo]);
          float pv[4], dv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = 4 * g4 + i;
            const int q = q0 + qo + i;
            float x = s[rr];
            float gcap = 1.0f;
            if constexpr (SOFTCAP) {
              x = transform_score<true>(x, p.softcap_pre, p.softcap);
              const float th = x * icap;
              gcap = fmaf(-th, th, 1.0f);
            }
            if constexpr (ALIBI) x = fmaf(-slope, fabsf((float)(q + off - key)), x);
            if constexpr (MASKED) {
              const bool vis = (q < sq) & (key < sk) & ((wr < 0) | (key <= q + off + wr)) &
                               ((wl < 0) | (key >= q + off - wl));
              x = vis ? x : -INFINITY;
            }
            const float pr = fast_exp2(fmaf(x, c2, -l4[i]));
            pv[i] = pr;
            if constexpr (DO_DK) {
              float d = pr * (dp[rr] - d4[i]);
              if constexpr (SOFTCAP) d *= gcap;
              dv[i] = d;
            }
          }
          if constexpr (DO_DV) {
            pp[2 * g4] = Ty::pack(pv[0], pv[1]);
            pp[2 * g4 + 1] = Ty::pack(pv[2], pv[3]);
          }
          if constexpr (DO_DK) {
            ps[2 * g4] = Ty::pack(dv[0], dv[1]);
            ps[2 * g4 + 1] = Ty::pack(dv[2], dv[3]);
          }
        }
        };
        if (full) elementwise(std::false_type{});
        else elementwise(std::true_type{});
        // dV^T += dO^T P and dK^T += Q^T dS over the block's two 16-query
        // slices, contracting in the order the score registers hold them.
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            if constexpr (DO_DV) {
              const u32x4 bp = {pp[4 * k2 + 0], pp[4 * k2 + 1], pp[4 * k2 + 2], pp[4 * k2 + 3]};
              const u32x4 a = TR_AHEAD ? tg[k2][dt] : tr_operand<D>(g_cur, oo, 2 * qb + k2, dt);
              acc_dv[dt] = Ty::mfma(a, bp, acc_dv[dt]);
            }
            if constexpr (DO_DK) {
              const u32x4 bs = {ps[4 * k2 + 0], ps[4 * k2 + 1], ps[4 * k2 + 2], ps[4 * k2 + 3]};
              const u32x4 a = TR_AHEAD ? tq[k2][dt] : tr_operand<D>(q_cur, oo, 2 * qb + k2, dt);
              acc_dk[dt] = Ty::mfma(a, bs, acc_dk[dt]);
            }
          }
        }
      }
    }
    if (r + 1 < n) stage_rows((r + 1) & 1);
    if (r + 2 < n) barrier_vmem_le<2 * Copier::LOADS>();
    else barrier_vmem_le<0>();
    h = h1;
    q0 = q1;
  };

  if (n > 0) {
    issue_rows(h, q0);
    issue(h, q0, lds_q0, lds_g0);
    if (n > 1) {
      int h1 = h, q1 = q0;
      advance(h1, q1);
      issue(h1, q1, lds_q1, lds_g1);
    }
    stage_rows(0);
    if (n > 1) barrier_vmem_le<2 * Copier::LOADS>();
    else barrier_vmem_le<0>();
    int r = 0;
    for (; r + 3 <= n; r += 3) {
      step(std::integral_constant<int, 0>{}, r);
      step(std::integral_constant<int, 1>{}, r + 1);
      step(std::integral_constant<int, 2>{}, r + 2);
    }
    if (r < n) step(std::integral_constant<int, 0>{}, r);
    if (r + 1 < n) step(std::integral_constant<int, 1>{}, r + 1);
  }

  // One pass: the gradients leave through the idle Q stage buffers (the last
  // step's barrier has retired every wave's reads of them); wave w takes
  // stage buffer w, dK in its first half and dV in its second.
  if constexpr (PASSES == 1 && NW <= 4) {
    if (n > 0 && rows_aligned16(p.dk, p.dk_batch, p.dk_row, p.dk_head) &&
        rows_aligned16(p.dv, p.dv_batch, p.dv_row, p.dv_head)) {
      char* region = wave == 0 ? lds_q0 : wave == 1 ? lds_q1 : wave == 2 ? lds_q2 : lds_g0;
      uint16_t* dk0 = reinterpret_cast<uint16_t*>(p.dk) + b * p.dk_batch + (int64_t)(sr.k_start + wk_lo) * p.dk_row +
                      kvh * p.dk_head;
      uint16_t* dv0 = reinterpret_cast<uint16_t*>(p.dv) + b * p.dv_batch + (int64_t)(sr.k_start + wk_lo) * p.dv_row +
                      kvh * p.dv_head;
      store_rows_staged<Ty, D>(region, acc_dk, p.scale, lane, [&](int rr) -> uint16_t* {
        return wk_lo + rr < sk ? dk0 + (int64_t)rr * p.dk_row : nullptr;
      });
      store_rows_staged<Ty, D>(region + TILEB / 2, acc_dv, 1.0f, lane, [&](int rr) -> uint16_t* {
        return wk_lo + rr < sk ? dv0 + (int64_t)rr * p.dv_row : nullptr;
      });
      return;
    }
  }
  if (key_valid) {
    if constexpr (DO_DK) {
      uint16_t* dkp = reinterpret_cast<uint16_t*>(p.dk) + b * p.dk_batch +
                      (int64_t)(sr.k_start + key) * p.dk_row + kvh * p.dk_head;
      store_rows<Ty, D>(dkp, acc_dk, p.scale, hl);
    }
    if constexpr (DO_DV) {
      uint16_t* dvp = reinterpret_cast<uint16_t*>(p.dv) + b * p.dv_batch +
                      (int64_t)(sr.k_start + key) * p.dv_row + kvh * p.dv_head;
      store_rows<Ty, D>(dvp, acc_dv, 1.0f, hl);
    }
  }
  };  // run_pass

  run_pass(std::integral_constant<int, 0>{});
  if constexpr (PASSES == 2) run_pass(std::integral_constant<int, 1>{});
}

// ---------------------------------------------------------------- dK, dV in wave pairs
// Eight waves, two per SIMD.  Waves w and w + 4 (one SIMD) own the same 32
// keys and split a step's four tile products between them:
//  * the P wave (w < 4) forms S = Q K^T and P = exp2(c s - LSE), accumulates
//    dV^T += dO^T P, and leaves P (times the softcap derivative g) packed to
//    16 bits in LDS, in its own register layout;
//  * the dS wave (w >= 4) runs one step behind: dP = dO V^T, then
//    dS = (P g)(dP - D) from that LDS copy, and dK^T += Q^T dS.
// A wave holds one gradient's accumulators and one of the K / V row sets, so
// two waves fit per SIMD without forming S twice, and the two roles' matrix
// and elementwise phases interleave on the SIMD.  dS is formed from the
// 16-bit P that the dV product also uses.  Q / dO tiles stream one step
// ahead into three stages: a step reads its own tiles (P wave) and the
// previous step's (dS wave).  Both waves of a pair derive the same mask and
// skip decisions from the pair's key range, so the dS wave reads exactly the
// steps the P wave wrote.
template <class Ty, int D, bool SOFTCAP, bool ALIBI>
__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_pair_kernel(const BwdKernelParams p) {
  constexpr int NW = 8, NT = 512, NP = 4;  // waves, threads, wave pairs
  constexpr int BQ = D > 128 ? 32 : 64;    // queries per step
  constexpr int QB = BQ / 32;              // 32-query MFMA blocks per step
  constexpr int BN = 32 * NP;              // keys per workgroup
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BQ * ROWB;
  constexpr int DS = D / 16;
  constexpr int DT = D / 32;
  using Copier = TileCopier<BQ, D, NT>;

  __shared__ __attribute__((aligned(16))) char lds_q0[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_q1[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_q2[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_g0[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_g1[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_g2[TILEB];
  // P hand-over: [step parity][pair][query block][half] of 64 lanes x 16 bytes.
  __shared__ __attribute__((aligned(16))) u32x4 lds_p[2][NP][QB][2][64];
  __shared__ __attribute__((aligned(16))) float lds_lse[3][BQ];
  __shared__ __attribute__((aligned(16))) float lds_dd[3][BQ];
  // At D = 256 the last NX fragments of each lane's K / V row sit in LDS (one
  // slot per wave, written once) rather than in VGPRs: held in registers they
  // overflowed the 256 available and were spilled, and a scratch reload, being
  // a vector-memory load, waits for every copy in flight before it.
  constexpr int NX = D > 128 ? 5 : 0;
  constexpr int NR = DS - NX;  // fragments held in VGPRs
  __shared__ __attribute__((aligned(16))) u32x4 lds_kx[NX > 0 ? NW * NX * 64 : 1];
  auto qbuf = [&](auto st) __attribute__((always_inline)) -> char* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return lds_q0;
    else if constexpr (S == 1) return lds_q1;
    else return lds_q2;
  };
  auto gbuf = [&](auto st) __attribute__((always_inline)) -> char* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return lds_g0;
    else if constexpr (S == 1) return lds_g1;
    else return lds_g2;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & (NP - 1);
  const bool p_wave = wave < NP;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  const TileRank tr = tile_rank();
  const int kvh = tr.head, b = tr.b;
  const SeqRange sr = seq_range(p, b);
  const int sq = sr.sq, sk = sr.sk, off = sk - sq;
  const int n0 = tr.rank * BN;
  if (n0 >= sk) return;
  const int wl = p.window_left, wr = p.window_right;
  const int G = p.group;

  // This lane's key and the pair's key range.
  const int wk_lo = n0 + 32 * pair;
  const int key = wk_lo + l32;
  const bool key_valid = key < sk;
  const int keyc = key_valid ? key : sk - 1;
  const bool wave_live = wk_lo < sk;
  const int wk_hi = min(sk - 1, wk_lo + 31);

  // Queries that see some key of this workgroup, walked per query head.
  const int wg_hi = min(sk - 1, n0 + BN - 1);
  const int q_lo = (wr >= 0) ? max(0, n0 - off - wr) : 0;
  const int q_hi = (wl >= 0) ? min(sq - 1, wg_hi - off + wl) : sq - 1;
  const int qblk_lo = q_lo / BQ;
  const int nsph = (q_hi >= q_lo) ? (q_hi / BQ + 1 - qblk_lo) : 0;
  const int n = G * nsph;

  OperandOffsets<D> oo;
  oo.init(lane);
  Copier cp;
  cp.init(wave, lane, NW);

  const float c2 = p.scale_log2;
  const float icap = p.inv_softcap;
  // Queries that see this lane's key: [qlo, qlo + qspan) (empty for a key past
  // the valid length), so a score is masked by one unsigned compare.
  const int qlo = (wr >= 0) ? max(0, key - off - wr) : 0;
  const int qhi = min(sq - 1, (wl >= 0) ? key - off + wl : 0x3fffffff);
  const uint32_t qspan = (key_valid && qhi >= qlo) ? (uint32_t)(qhi - qlo + 1) : 0u;

  auto advance = [&](int& h, int& q0) __attribute__((always_inline)) {
    q0 += BQ;
    if (q0 >= (qblk_lo + nsph) * BQ) {
      q0 = qblk_lo * BQ;
      ++h;
    }
  };
  auto issue = [&](int h, int q0, char* qt, char* gt) __attribute__((always_inline)) {
    const char* qb = reinterpret_cast<const char*>(p.q) +
                     2 * (b * p.q_batch + (int64_t)(sr.q_start + q0) * p.q_row + h * p.q_head);
    const char* gb = reinterpret_cast<const char*>(p.dout) +
                     2 * (b * p.do_batch + (int64_t)(sr.q_start + q0) * p.do_row + h * p.do_head);
    cp.copy(qb, 2 * p.q_row, sq - q0, qt, wave, NW);
    cp.copy(gb, 2 * p.do_row, sq - q0, gt, wave, NW);
  };
  // LSE / D rows of a step: loaded by the first BQ threads (P waves) one step
  // ahead, staged to LDS slot (step % 3) at the end of the step before.
  float st_lse = 0.0f, st_dd = 0.0f;
  auto issue_rows = [&](int h, int q0) __attribute__((always_inline)) {
    if (tid < BQ) {
      const int q = q0 + tid;
      const int64_t li = b * p.lse_batch + (int64_t)h * p.lse_head + sr.q_start + q;
      st_lse = q < sq ? p.lse[li] : -INFINITY;
      st_dd = q < sq ? p.dsum[li] : 0.0f;
    }
  };
  auto stage_rows = [&](int slot) __attribute__((always_inline)) {
    if (tid < BQ) {
      lds_lse[slot][tid] = lse_to_exp2(st_lse);
      lds_dd[slot][tid] = st_dd;
    }
  };
  // Does the pair see any (query, key) of the step at q0?  And all of them?
  auto sees = [&](int q0) __attribute__((always_inline)) -> bool {
    const int qv_hi = min(sq - 1, q0 + BQ - 1);
    return wave_live && (wr < 0 || wk_lo <= qv_hi + off + wr) && (wl < 0 || wk_hi >= q0 + off - wl);
  };
  auto full_step = [&](int q0) __attribute__((always_inline)) -> bool {
    return q0 + BQ - 1 < sq && wk_lo + 31 < sk && (wr < 0 || wk_lo + 31 <= q0 + off + wr) &&
           (wl < 0 || wk_lo >= q0 + BQ - 1 + off - wl);
  };
  // A = rows of a 32-query block of an LDS tile, B = the lane's K or V row
  // fragments: S (or dP) of the block, operand reads one MFMA ahead.
  auto rows_product = [&](const char* tile, const u32x4 (&bf)[NR]) __attribute__((always_inline)) -> f32x16 {
    f32x16 acc = f32x16{};
    u32x4 cur = *reinterpret_cast<const u32x4*>(tile + oo.row_off(0));
#pragma unroll
    for (int t = 0; t < DS; ++t) {
      u32x4 nxt = cur;
      if (t + 1 < DS) nxt = *reinterpret_cast<const u32x4*>(tile + oo.row_off(t + 1));
      if constexpr (NX > 0) {
        const u32x4 bt = t < NR ? bf[t < NR ? t : 0] : lds_kx[(wave * NX + (t - NR)) * 64 + lane];
        acc = Ty::mfma(cur, bt, acc);
      } else {
        acc = Ty::mfma(cur, bf[t], acc);
      }
      cur = nxt;
    }
    return acc;
  };
  // acc^T += tile^T B over the block's two 16-query slices (A read transposed),
  // operands one MFMA ahead; B = the packed 16-bit P or dS of the block.
  auto tr_product = [&](const char* tile, int qb, const uint32_t (&pk)[8], f32x16 (&acc)[DT])
                        __attribute__((always_inline)) {
    constexpr int NOP = 2 * DT;
    u32x4 cur = tr_operand<D>(tile, oo, 2 * qb, 0);
#pragma unroll
    for (int i = 0; i < NOP; ++i) {
      const int k2 = i / DT, dt = i % DT;
      u32x4 nxt = cur;
      if (i + 1 < NOP) nxt = tr_operand<D>(tile, oo, 2 * qb + (i + 1) / DT, (i + 1) % DT);
      const u32x4 bop = {pk[4 * k2 + 0], pk[4 * k2 + 1], pk[4 * k2 + 2], pk[4 * k2 + 3]};
      acc[dt] = Ty::mfma(cur, bop, acc[dt]);
      cur = nxt;
    }
  };

  f32x16 acc[DT];  // dV^T (P waves) or dK^T (dS waves)
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  if (n > 0) {
    // The key's K row (P waves) or V row (dS waves), loaded before the first
    // stage's wait so that it has arrived when the walk starts: a load still
    // in flight at the loop entry would make the first step of every unrolled
    // iteration wait for all outstanding copies, the next stage's included.
    u32x4 kvf[NR];
    [[maybe_unused]] u32x4 kvx[NX > 0 ? NX : 1];
    {
      const uint16_t* rp =
          p_wave ? reinterpret_cast<const uint16_t*>(p.k) + b * p.k_batch + (int64_t)(sr.k_start + keyc) * p.k_row +
                       kvh * p.k_head
                 : reinterpret_cast<const uint16_t*>(p.v) + b * p.v_batch + (int64_t)(sr.k_start + keyc) * p.v_row +
                       kvh * p.v_head;
#pragma unroll
      for (int t = 0; t < NR; ++t) kvf[t] = *reinterpret_cast<const u32x4*>(rp + 16 * t + 8 * hl);
#pragma unroll
      for (int t = NR; t < DS; ++t) kvx[t - NR] = *reinterpret_cast<const u32x4*>(rp + 16 * t + 8 * hl);
    }
    // The ALiBi slope of the first step's query head, loaded before the same
    // wait; each step then loads the next step's slope before its copies, so
    // no slope load is outstanding behind them when the scores need it.
    [[maybe_unused]] float slope_raw = 0.0f;
    if constexpr (ALIBI) slope_raw = p.alibi[b * p.alibi_bstride + kvh * G];
    {
      const int h = kvh * G, q0 = qblk_lo * BQ;
      issue_rows(h, q0);
      issue(h, q0, lds_q0, lds_g0);
      stage_rows(0);
      barrier_vmem_le<0>();
    }
    // Only this wave reads its slot, and its LDS accesses complete in order.
#pragma unroll
    for (int x = 0; x < NX; ++x) lds_kx[(wave * NX + x) * 64 + lane] = kvx[x];
    if (p_wave) {
      const u32x4(&kf)[NR] = kvf;
      int h = kvh * G, q0 = qblk_lo * BQ;
      // Step r computes on stage ST = r % 3 and fills stage (r + 1) % 3.
      auto step = [&](auto stc, int r) __attribute__((always_inline)) {
        constexpr int ST = decltype(stc)::value;
        constexpr int FILL = (ST + 1) % 3;
        int h1 = h, q1 = q0;
        advance(h1, q1);
        [[maybe_unused]] float slope_raw_next = 0.0f;
        if (r + 1 < n) {
          if constexpr (ALIBI) slope_raw_next = p.alibi[b * p.alibi_bstride + h1];
          issue_rows(h1, q1);
          issue(h1, q1, qbuf(std::integral_constant<int, FILL>{}), gbuf(std::integral_constant<int, FILL>{}));
        }
        if (r < n && sees(q0)) {
          const char* q_cur = qbuf(stc);
          const char* g_cur = gbuf(stc);
          float slope = 0.0f;
          if constexpr (ALIBI) slope = slope_raw * p.alibi_inv_scale;
          const bool full = full_step(q0);
          // S of every 32-query block first, then each block's P, hand-over and dV.
          f32x16 sb[QB];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sb[qb] = rows_product(q_cur + qb * 32 * ROWB, kf);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const f32x16& s = sb[qb];
            uint32_t pp[8];
            [[maybe_unused]] uint32_t pg[8];
            auto elementwise = [&](auto masked_c) __attribute__((always_inline)) {
              constexpr bool MASKED = decltype(masked_c)::value;
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4) {
                const int qo = 32 * qb + 8 * g4 + 4 * hl;
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lds_lse[ST][qo]);
                float pv[4], gv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int q = q0 + qo + i;
                  float x = s[4 * g4 + i];
                  float gcap = 1.0f;
                  if constexpr (SOFTCAP) {
                    x = transform_score<true>(x, p.softcap_pre, p.softcap);
                    const float th = x * icap;
                    gcap = fmaf(-th, th, 1.0f);
                  }
                  if constexpr (ALIBI) x = fmaf(-slope, fabsf((float)(q + off - key)), x);
                  if constexpr (MASKED) x = (uint32_t)(q - qlo) < qspan ? x : -INFINITY;
                  pv[i] = fast_exp2(fmaf(x, c2, -l4[i]));
                  gv[i] = pv[i] * gcap;
                }
                pp[2 * g4] = Ty::pack(pv[0], pv[1]);
                pp[2 * g4 + 1] = Ty::pack(pv[2], pv[3]);
                if constexpr (SOFTCAP) {
                  pg[2 * g4] = Ty::pack(gv[0], gv[1]);
                  pg[2 * g4 + 1] = Ty::pack(gv[2], gv[3]);
                }
              }
            };
            if (full) elementwise(std::false_type{});
            else elementwise(std::true_type{});
            if constexpr (SOFTCAP) {
              lds_p[r & 1][pair][qb][0][lane] = u32x4{pg[0], pg[1], pg[2], pg[3]};
              lds_p[r & 1][pair][qb][1][lane] = u32x4{pg[4], pg[5], pg[6], pg[7]};
            } else {
              lds_p[r & 1][pair][qb][0][lane] = u32x4{pp[0], pp[1], pp[2], pp[3]};
              lds_p[r & 1][pair][qb][1][lane] = u32x4{pp[4], pp[5], pp[6], pp[7]};
            }
            tr_product(g_cur, qb, pp, acc);
          }
        }
        if (r + 1 < n) stage_rows(FILL);
        barrier_vmem_le<0>();
        h = h1;
        q0 = q1;
        if constexpr (ALIBI) slope_raw = slope_raw_next;
      };
      int r = 0;
      for (; r + 3 <= n + 1; r += 3) {
        step(std::integral_constant<int, 0>{}, r);
        step(std::integral_constant<int, 1>{}, r + 1);
        step(std::integral_constant<int, 2>{}, r + 2);
      }
      if (r < n + 1) step(std::integral_constant<int, 0>{}, r);
      if (r + 1 < n + 1) step(std::integral_constant<int, 1>{}, r + 1);
    } else {
      const u32x4(&vf)[NR] = kvf;
      int h = kvh * G, q0 = qblk_lo * BQ;  // position of step r
      int qp = q0;                          // position of step r - 1
      f32x16 db[QB];                        // dP of the blocks of a step
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) db[qb] = f32x16{};
      auto form_dp = [&](const char* g_tile) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) db[qb] = rows_product(g_tile + qb * 32 * ROWB, vf);
      };
      // dS = P (dP - D) of step r - 1 from db and the P the P wave handed over,
      // then dK^T += Q^T dS.
      // P and D of step r - 1, read from LDS ahead of the dP MFMAs (D = 64 / 128 order).
      u32x4 pre_p[QB][2];
      f32x4 pre_d[QB][4];
      auto load_pd = [&](int r, const float* dd_prev) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          pre_p[qb][0] = lds_p[(r - 1) & 1][pair][qb][0][lane];
          pre_p[qb][1] = lds_p[(r - 1) & 1][pair][qb][1][lane];
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            pre_d[qb][g4] = *reinterpret_cast<const f32x4*>(&dd_prev[32 * qb + 8 * g4 + 4 * hl]);
        }
      };
      auto finish = [&](int r, const char* q_prev, const float* dd_prev, auto pre_c) __attribute__((always_inline)) {
        constexpr bool PRE = decltype(pre_c)::value;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const f32x16& dp = db[qb];
          u32x4 h0, h1v;
          if constexpr (PRE) {
            h0 = pre_p[qb][0];
            h1v = pre_p[qb][1];
          } else {
            h0 = lds_p[(r - 1) & 1][pair][qb][0][lane];
            h1v = lds_p[(r - 1) & 1][pair][qb][1][lane];
          }
          const uint32_t ph[8] = {h0[0], h0[1], h0[2], h0[3], h1v[0], h1v[1], h1v[2], h1v[3]};
          uint32_t ps[8];
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int qo = 32 * qb + 8 * g4 + 4 * hl;
            f32x4 d4;
            if constexpr (PRE) d4 = pre_d[qb][g4];
            else d4 = *reinterpret_cast<const f32x4*>(&dd_prev[qo]);
            const f32x2 pa = unpack2<Ty>(ph[2 * g4]);
            const f32x2 pb = unpack2<Ty>(ph[2 * g4 + 1]);
            ps[2 * g4] = Ty::pack(pa[0] * (dp[4 * g4 + 0] - d4[0]), pa[1] * (dp[4 * g4 + 1] - d4[1]));
            ps[2 * g4 + 1] = Ty::pack(pb[0] * (dp[4 * g4 + 2] - d4[2]), pb[1] * (dp[4 * g4 + 3] - d4[3]));
          }
          tr_product(q_prev, qb, ps, acc);
        }
      };
      // At head_dim 256 step r first finishes step r - 1 (its dP carried over
      // the barrier) and then forms dP of step r, so its dS arithmetic runs
      // under the P wave's S MFMAs and its dK MFMAs under the P wave's
      // exponentials (+2%).  At 64 / 128 that order measured 1% slower, so
      // there step r forms dP of step r - 1 and finishes it at once.
      constexpr bool CARRY = D > 128;
      bool carried = false;  // CARRY: db holds dP of step r - 1
      auto step = [&](auto stc, int r) __attribute__((always_inline)) {
        constexpr int ST = decltype(stc)::value;
        constexpr int FILL = (ST + 1) % 3;
        constexpr int PREV = (ST + 2) % 3;
        int h1 = h, q1 = q0;
        advance(h1, q1);
        if (r + 1 < n) issue(h1, q1, qbuf(std::integral_constant<int, FILL>{}), gbuf(std::integral_constant<int, FILL>{}));
        if constexpr (CARRY) {
          if (carried) finish(r, qbuf(std::integral_constant<int, PREV>{}), lds_dd[PREV], std::false_type{});
          carried = r < n && sees(q0);
          if (carried) form_dp(gbuf(stc));
        } else {
          if (r >= 1 && sees(qp)) {
            load_pd(r, lds_dd[PREV]);
            form_dp(gbuf(std::integral_constant<int, PREV>{}));
            finish(r, qbuf(std::integral_constant<int, PREV>{}), lds_dd[PREV], std::true_type{});
          }
        }
        barrier_vmem_le<0>();
        qp = q0;
        h = h1;
        q0 = q1;
      };
      int r = 0;
      for (; r + 3 <= n + 1; r += 3) {
        step(std::integral_constant<int, 0>{}, r);
        step(std::integral_constant<int, 1>{}, r + 1);
        step(std::integral_constant<int, 2>{}, r + 2);
      }
      if (r < n + 1) step(std::integral_constant<int, 0>{}, r);
      if (r + 1 < n + 1) step(std::integral_constant<int, 1>{}, r + 1);
    }
  }

  // dV (P waves) and dK (dS waves) leave through the idle Q / dO stage
  // buffers when eight 32-row blocks fit them (the last step's barrier has
  // retired every read of them).
  uint16_t* dst0;
  float mul;
  if (p_wave) {
    dst0 = reinterpret_cast<uint16_t*>(p.dv) + b * p.dv_batch + (int64_t)(sr.k_start + wk_lo) * p.dv_row +
           kvh * p.dv_head;
    mul = 1.0f;
  } else {
    dst0 = reinterpret_cast<uint16_t*>(p.dk) + b * p.dk_batch + (int64_t)(sr.k_start + wk_lo) * p.dk_row +
           kvh * p.dk_head;
    mul = p.scale;
  }
  const int64_t drow = p_wave ? p.dv_row : p.dk_row;
  constexpr int REGB = 32 * ROWB;
  constexpr int RPBUF = TILEB / REGB;  // 32-row blocks per stage buffer
  if constexpr (6 * RPBUF >= NW) {
    if (n > 0 && rows_aligned16(p.dk, p.dk_batch, p.dk_row, p.dk_head) &&
        rows_aligned16(p.dv, p.dv_batch, p.dv_row, p.dv_head)) {
      const int bi = wave / RPBUF;
      char* base = bi == 0 ? lds_q0 : bi == 1 ? lds_q1 : bi == 2 ? lds_q2 : bi == 3 ? lds_g0 : bi == 4 ? lds_g1 : lds_g2;
      store_rows_staged<Ty, D>(base + (wave % RPBUF) * REGB, acc, mul, lane, [&](int rr) -> uint16_t* {
        return wk_lo + rr < sk ? dst0 + (int64_t)rr * drow : nullptr;
      });
      return;
    }
  }
  if (key_valid) store_rows<Ty, D>(dst0 + (int64_t)l32 * drow, acc, mul, hl);
}

// ---------------------------------------------------------------- dQ
// NW waves of 32 queries, WPE waves per SIMD (2; 1 at D = 256, where the Q
// and dO fragments and the dQ accumulators alone take 256 registers).
template <class Ty, int D, bool SOFTCAP, bool ALIBI, int NW = 4, int WPE = 2>
__global__ void __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64), amdgpu_waves_per_eu(WPE, WPE)))
bwd_dq_kernel(const BwdKernelParams p) {
  constexpr int NT = NW * 64;
  constexpr int BK = 64;            // keys per step
  constexpr int BQ = 32 * NW;       // queries per workgroup
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BK * ROWB;
  constexpr int KT = BK / 32;
  constexpr int DS = D / 16;
  constexpr int DT = D / 32;
  constexpr int KS = BK / 16;
  constexpr int LEAD = 4;
  using Copier = TileCopier<BK, D, NT>;

  __shared__ __attribute__((aligned(16))) char lds_k0[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_k1[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_v0[TILEB];
  __shared__ __attribute__((aligned(16))) char lds_v1[TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  const TileRank tr = tile_rank();
  const int head = tr.head, b = tr.b;
  const SeqRange sr = seq_range(p, b);
  const int sq = sr.sq, sk = sr.sk, off = sk - sq;
  const int m0 = ((int)gridDim.x - 1 - tr.rank) * BQ;  // the last query tiles see the most keys
  if (m0 >= sq) return;
  const int kvh = head / p.group;
  const int wl = p.window_left, wr = p.window_right;

  const int row = m0 + 32 * wave + l32;
  const bool q_valid = row < sq;
  const int rowc = q_valid ? row : sq - 1;
  const int kmin = (wl >= 0) ? row + off - wl : -0x40000000;
  const int kmax = min(sk - 1, (wr >= 0) ? row + off + wr : 0x3fffffff);
  const int wrow_lo = m0 + 32 * wave;
  const int wrow_hi = min(sq - 1, wrow_lo + 31);
  const bool wave_live = wrow_lo < sq;
  const int wk_lo = (wl >= 0) ? wrow_lo + off - wl : -0x40000000;
  const int wk_hi = min(sk - 1, (wr >= 0) ? wrow_hi + off + wr : 0x3fffffff);
  const int full_lo = (wl >= 0) ? wrow_hi + off - wl : -0x40000000;
  const int full_hi = min(sk - 1, (wr >= 0) ? wrow_lo + off + wr : 0x3fffffff);

  // KV steps of the tile.
  const int row_hi = min(sq - 1, m0 + BQ - 1);
  const int n_lo = (wl >= 0) ? max(0, m0 + off - wl) : 0;
  const int n_hi = (wr >= 0) ? min(sk, row_hi + off + wr + 1) : sk;
  const int blk_lo = n_lo / BK;
  const int n = (n_hi > n_lo) ? (n_hi + BK - 1) / BK - blk_lo : 0;

  // Q and dO rows of this lane's query: B operands.
  u32x4 qf[DS], gf[DS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + b * p.q_batch +
                         (int64_t)(sr.q_start + rowc) * p.q_row + head * p.q_head;
    const uint16_t* gp = reinterpret_cast<const uint16_t*>(p.dout) + b * p.do_batch +
                         (int64_t)(sr.q_start + rowc) * p.do_row + head * p.do_head;
#pragma unroll
    for (int t = 0; t < DS; ++t) {
      qf[t] = *reinterpret_cast<const u32x4*>(qp + 16 * t + 8 * hl);
      gf[t] = *reinterpret_cast<const u32x4*>(gp + 16 * t + 8 * hl);
    }
  }
  const int64_t li = b * p.lse_batch + (int64_t)head * p.lse_head + sr.q_start + rowc;
  const float lse_row = p.lse[li];  // unconditional (rowc is a valid row): no wait before the loads below
  const float lse2 = q_valid ? lse_to_exp2(lse_row) : INFINITY;
  // The O rows of this lane's query (the dO fragments' chunks), for D below.
  u32x4 of[DS];
  {
    const uint16_t* op = reinterpret_cast<const uint16_t*>(p.o) + b * p.o_batch +
                         (int64_t)(sr.q_start + rowc) * p.o_row + head * p.o_head;
#pragma unroll
    for (int t = 0; t < DS; ++t) of[t] = *reinterpret_cast<const u32x4*>(op + 16 * t + 8 * hl);
  }
  float dd = 0.0f;
  float slope = 0.0f;
  if constexpr (ALIBI) slope = p.alibi[b * p.alibi_bstride + head] * p.alibi_inv_scale;

  OperandOffsets<D> oo;
  oo.init(lane);
  Copier cp;
  cp.init(wave, lane, NW);
  const char* kbase = reinterpret_cast<const char*>(p.k) +
                      2 * (b * p.k_batch + (int64_t)sr.k_start * p.k_row + kvh * p.k_head);
  const char* vbase = reinterpret_cast<const char*>(p.v) +
                      2 * (b * p.v_batch + (int64_t)sr.k_start * p.v_row + kvh * p.v_head);
  auto issue = [&](int blk, char* kt, char* vt) __attribute__((always_inline)) {
    const int j0 = blk * BK;
    cp.copy(kbase + (int64_t)j0 * 2 * p.k_row, 2 * p.k_row, sk - j0, kt, wave, NW);
    cp.copy(vbase + (int64_t)j0 * 2 * p.v_row, 2 * p.v_row, sk - j0, vt, wave, NW);
  };

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  const float c2 = p.scale_log2;
  const float icap = p.inv_softcap;

  auto step = [&](auto stc, int r) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
    char* k_cur = ST == 0 ? lds_k0 : lds_k1;
    char* v_cur = ST == 0 ? lds_v0 : lds_v1;
    const int blk = blk_lo + r;
    if (r + 1 < n) issue(blk + 1, ST == 0 ? lds_k1 : lds_k0, ST == 0 ? lds_v1 : lds_v0);
    const int j0 = blk * BK;
    if (wave_live && j0 <= wk_hi && j0 + BK - 1 >= wk_lo) {
      f32x16 s[KT], dp[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[kt] = f32x16{};
        dp[kt] = f32x16{};
      }
#pragma unroll
      for (int t = 0; t < DS; ++t) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(k_cur + kt * 32 * ROWB + oo.row_off(t));
          s[kt] = Ty::mfma(a, qf[t], s[kt]);
          const u32x4 a2 = *reinterpret_cast<const u32x4*>(v_cur + kt * 32 * ROWB + oo.row_off(t));
          dp[kt] = Ty::mfma(a2, gf[t], dp[kt]);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, LEAD, 0);
      for (int i = 0; i < 2 * DS * KT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      // dS^T in place of the scores, then (only on steps that an edge crosses
      // for the wave) zero where the key is not visible: P = 0 there, and a
      // select drops whatever the unmasked formula gave (inf or NaN included).
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          float x = s[kt][rr];
          float gcap = 1.0f;
          if constexpr (SOFTCAP) {
            x = transform_score<true>(x, p.softcap_pre, p.softcap);
            const float th = x * icap;
            gcap = fmaf(-th, th, 1.0f);
          }
          if constexpr (ALIBI) {
            const int kk = j0 + 32 * kt + 8 * (rr >> 2) + 4 * hl + (rr & 3);
            x = fmaf(-slope, fabsf((float)(row + off - kk)), x);
          }
          const float pr = fast_exp2(fmaf(x, c2, -lse2));
          float d = pr * (dp[kt][rr] - dd);
          if constexpr (SOFTCAP) d *= gcap;
          s[kt][rr] = d;
        }
      }
      if (!(j0 >= full_lo && j0 + BK - 1 <= full_hi)) {
        // key - kmin in [0, kmax - kmin] as one unsigned compare
        const uint32_t span = (uint32_t)(kmax - kmin);
        const int base = j0 + 4 * hl - kmin;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const uint32_t rel = (uint32_t)(base + 32 * kt + 8 * (rr >> 2) + (rr & 3));
            s[kt][rr] = rel <= span ? s[kt][rr] : 0.0f;
          }
      }
      uint32_t ps[KT][8];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r2 = 0; r2 < 16; r2 += 2) ps[kt][r2 >> 1] = Ty::pack(s[kt][r2], s[kt][r2 + 1]);
      // dQ^T += K^T dS^T, contracting over the step's keys in register order.
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 bs = {ps[ks >> 1][4 * (ks & 1) + 0], ps[ks >> 1][4 * (ks & 1) + 1],
                          ps[ks >> 1][4 * (ks & 1) + 2], ps[ks >> 1][4 * (ks & 1) + 3]};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = Ty::mfma(tr_operand<D>(k_cur, oo, ks, dt), bs, acc[dt]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * LEAD, 0);
      for (int i = 0; i < KS * DT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
    wait_vmem();
    __syncthreads();
  };

  if (n > 0) issue(blk_lo, lds_k0, lds_v0);
  wait_vmem();  // Q, dO, O and the first K/V tile: one latency for all of them
  // D of this lane's query, <dO, O> in fp32: lanes l and l + 32 hold the two
  // halves of the row, so their partial sums meet in one swap; both lanes add
  // the same two values and agree bit for bit.
  {
    float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < DS; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 a = unpack2<Ty>(of[t][i]);
        const f32x2 g = unpack2<Ty>(gf[t][i]);
        part[i] = fmaf(a[1], g[1], fmaf(a[0], g[0], part[i]));
      }
    const float half = (part[0] + part[1]) + (part[2] + part[3]);
    const float whole = half + __shfl_xor(half, 32);
    if (q_valid) {
      dd = whole;
      if (hl == 0) p.dsum[li] = whole;  // for the dK/dV kernel
    }
  }
  if (n > 0) {
    // The copies have landed (wait above); only the D store may still be in
    // flight, and nothing in this kernel reads it.
    barrier_vmem_le<1>();
    int r = 0;
    for (; r + 2 <= n; r += 2) {
      step(std::integral_constant<int, 0>{}, r);
      step(std::integral_constant<int, 1>{}, r + 1);
    }
    if (r < n) step(std::integral_constant<int, 0>{}, r);
  }

  // dQ leaves through the idle K/V stage buffers (the last step's barrier has
  // retired every wave's reads of them): two 32-row blocks per buffer.
  if (n > 0 && rows_aligned16(p.dq, p.dq_batch, p.dq_row, p.dq_head)) {
    constexpr int REGB = 32 * ROWB;
    static_assert(TILEB == 2 * REGB && NW <= 8, "two wave blocks per stage buffer");
    const int bi = wave >> 1;
    char* region = (bi == 0 ? lds_k0 : bi == 1 ? lds_k1 : bi == 2 ? lds_v0 : lds_v1) + (wave & 1) * REGB;
    uint16_t* dq0 = reinterpret_cast<uint16_t*>(p.dq) + b * p.dq_batch + (int64_t)(sr.q_start + wrow_lo) * p.dq_row +
                    head * p.dq_head;
    store_rows_staged<Ty, D>(region, acc, p.scale, lane, [&](int rr) -> uint16_t* {
      return wrow_lo + rr < sq ? dq0 + (int64_t)rr * p.dq_row : nullptr;
    });
    return;
  }
  if (q_valid) {
    uint16_t* dqp = reinterpret_cast<uint16_t*>(p.dq) + b * p.dq_batch + (int64_t)(sr.q_start + row) * p.dq_row +
                    head * p.dq_head;
    store_rows<Ty, D>(dqp, acc, p.scale, hl);
  }
}

// Kernel-shape overrides of the debug build (attn_debug_set_variants; the
// release library compiles none of them): 1 = dK/dV in two passes at 8
// waves (head_dim 64 / 128); 2 / 3 = dQ with 8 / 4 waves (256 / 128 queries
// per workgroup); 4 = dK/dV at one wave per SIMD (4 waves: one pass at head_dim
// 64 / 128, two walks at 256).

// dQ first (it also forms D, which the dK/dV kernel reads), then dK/dV; a
// kernel whose grid would be empty (no queries, or no keys) is not launched.
template <class Ty, int D, bool SOFTCAP, bool ALIBI>
hipError_t launch_bwd_t(const BwdKernelParams& p, hipStream_t stream) {
  if constexpr (D > 128) {
    // D = 256: the paired dK/dV kernel with 32-query steps (each wave's one
    // gradient and one K / V row set fill its 256 registers; a few values
    // spill to scratch, still 29% faster than two walks at one wave per SIMD,
    // which debug override 4 selects), and dQ at one wave per SIMD -- the Q and
    // dO rows and the dQ accumulators alone take 256 registers.
    if (p.seqlen_q > 0) {
      const dim3 grid((unsigned)((p.seqlen_q + 127) / 128), p.heads_q, p.batch);
      hipLaunchKernelGGL((bwd_dq_kernel<Ty, D, SOFTCAP, ALIBI, 4, 1>), grid, dim3(256), 0, stream, p);
    }
    if (p.seqlen_k > 0) {
      const dim3 grid((unsigned)((p.seqlen_k + 127) / 128), p.heads_kv, p.batch);
      bool launched = false;
      if constexpr (kDebugBuild) {
        if (bwd_variant() == 4) {
          hipLaunchKernelGGL((bwd_dkdv_kernel<Ty, D, SOFTCAP, ALIBI, 4, 1, 2>), grid, dim3(256), 0, stream, p);
          launched = true;
        }
      }
      if (!launched)
        hipLaunchKernelGGL((bwd_dkdv_pair_kernel<Ty, D, SOFTCAP, ALIBI>), grid, dim3(512), 0, stream, p);
    }
  } else {
    if (p.seqlen_q > 0) {
      // 256 queries per workgroup (8 waves, two per SIMD; half the K/V re-reads
      // from L2) when that grid gives every CU two workgroups, else 128
      // (twice the workgroups); the debug build's variant 2 forces 256, 3 forces 128.
      const int64_t wgs256 = (int64_t)((p.seqlen_q + 255) / 256) * p.heads_q * p.batch;
      const int v = kDebugBuild ? bwd_variant() : 0;
      if (v == 2 || (v != 3 && wgs256 >= 2 * (int64_t)compute_units())) {
        const dim3 grid((unsigned)((p.seqlen_q + 255) / 256), p.heads_q, p.batch);
        hipLaunchKernelGGL((bwd_dq_kernel<Ty, D, SOFTCAP, ALIBI, 8>), grid, dim3(512), 0, stream, p);
      } else {
        const dim3 grid((unsigned)((p.seqlen_q + 127) / 128), p.heads_q, p.batch);
        hipLaunchKernelGGL((bwd_dq_kernel<Ty, D, SOFTCAP, ALIBI>), grid, dim3(256), 0, stream, p);
      }
    }
    if (p.seqlen_k > 0) {
      // Default: the paired kernel (eight waves, two per SIMD; 128 keys per
      // workgroup).  Debug overrides: 1 = two passes at eight waves (256 keys),
      // 4 = one pass at one wave per SIMD (four waves, 128 keys).
      bool launched = false;
      if constexpr (kDebugBuild) {
        if (bwd_variant() == 1) {
          const dim3 grid((unsigned)((p.seqlen_k + 255) / 256), p.heads_kv, p.batch);
          hipLaunchKernelGGL((bwd_dkdv_kernel<Ty, D, SOFTCAP, ALIBI, 8, 2, 2>), grid, dim3(512), 0, stream, p);
          launched = true;
        } else if (bwd_variant() == 4) {
          const dim3 grid((unsigned)((p.seqlen_k + 127) / 128), p.heads_kv, p.batch);
          hipLaunchKernelGGL((bwd_dkdv_kernel<Ty, D, SOFTCAP, ALIBI, 4, 1, 1>), grid, dim3(256), 0, stream, p);
          launched = true;
        }
      }
      if (!launched) {
        const dim3 grid((unsigned)((p.seqlen_k + 127) / 128), p.heads_kv, p.batch);
        hipLaunchKernelGGL((bwd_dkdv_pair_kernel<Ty, D, SOFTCAP, ALIBI>), grid, dim3(512), 0, stream, p);
      }
    }
  }
  return hipGetLastError();
}

template <class Ty, int D>
hipError_t launch_bwd_d(const BwdKernelParams& p, hipStream_t stream) {
  const bool cap = p.softcap > 0.0f, al = p.alibi != nullptr;
  if (cap) return al ? launch_bwd_t<Ty, D, true, true>(p, stream) : launch_bwd_t<Ty, D, true, false>(p, stream);
  return al ? launch_bwd_t<Ty, D, false, true>(p, stream) : launch_bwd_t<Ty, D, false, false>(p, stream);
}

template <class Ty>
hipError_t launch_bwd_ty(const BwdKernelParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 64) return launch_bwd_d<Ty, 64>(p, stream);
  if (head_dim == 128) return launch_bwd_d<Ty, 128>(p, stream);
  if (head_dim == 256) return launch_bwd_d<Ty, 256>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace

#if !defined(ATTN_TU_DTYPE) || ATTN_TU_DTYPE == 0
hipError_t launch_bwd_f16(const BwdKernelParams& p, int head_dim, hipStream_t stream) {
  return launch_bwd_ty<TypeF16>(p, head_dim, stream);
}
#endif
#if !defined(ATTN_TU_DTYPE) || ATTN_TU_DTYPE == 1
hipError_t launch_bwd_bf16(const BwdKernelParams& p, int head_dim, hipStream_t stream) {
  return launch_bwd_ty<TypeBF16>(p, head_dim, stream);
}
#endif

}  // namespace attn
