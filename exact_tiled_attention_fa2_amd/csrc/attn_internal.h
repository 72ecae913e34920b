// Internal interface between the host C-ABI layer (attn_api.cpp) and the
// HIP kernels (attn_kernels.hip, attn_bwd.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Everything one launch of the tile kernel needs, resolved on the host.
// Strides are in elements.  Sequence offsets come from cu_seqlens (varlen) or
// are zero (dense / kv-cache).
struct FwdKernelParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // may be null
  float* o_part;       // split-KV partial outputs [splits][B][Hq][Sq][D] (null: write o)
  float* lse_part;     // split-KV partial LSEs    [splits][B][Hq][Sq]
  const int32_t* cu_seqlens_q;  // varlen prefix sums [B+1] (null: dense)
  const int32_t* cu_seqlens_k;
  const int32_t* seqused_k;     // kv-cache valid lengths [B] (null: seqlen_k)
  const int32_t* block_table;   // paged cache: page of (b, key / page_size) (null: contiguous)
  int32_t bt_stride, page_size, num_pages;  // paged cache; k_batch / v_batch = page stride
  int64_t q_batch, q_row, q_head;
  int64_t k_batch, k_row, k_head;
  int64_t v_batch, v_row, v_head;
  int64_t o_batch, o_row, o_head;
  int64_t lse_batch, lse_head;  // LSE index = b*lse_batch + h*lse_head + (q_start + row)
  int32_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, group;
  int32_t pack_gqa;     // 1: a query tile holds (row, head-in-group) pairs of one KV head
  int32_t num_splits;
  int32_t num_m_tiles;  // query tiles per (batch, head) in the grid's x dimension (set by the launcher)
  int32_t col_group;    // (head, batch) columns per longest-first group (set by the launcher)
  int32_t xcd_chunk;    // columns dealt to the XCDs in chunks of this many (set by the launcher)
  int32_t window_left, window_right;  // -1 unbounded; causal already folded into window_right
  float scale_log2;     // factor of the raw score inside exp2: scale*log2(e), or log2(e) with softcap
  float scale_ln;       // running max -> natural-log units: scale, or 1 with softcap
  float softcap_pre;    // scale / softcap
  float softcap;        // 0: off
  float tau;            // rescale threshold, log2 units
  const float* alibi;   // ALiBi slopes (null: off), slope(b, h) = alibi[b * alibi_bstride + h]
  int64_t alibi_bstride;
  float alibi_inv_scale;  // 1 / scale_ln: bias in raw-score units
  // Debug build only (null otherwise): per query row, 4 words at the LSE
  // index: live KV steps that set the first max, steps that skipped the
  // rescale, steps that rescaled, and the bits of the largest fp32 P formed.
  uint32_t* row_stats;
};

struct CombineParams {
  const float* o_part;
  const float* lse_part;
  void* o;
  float* lse;
  int64_t o_batch, o_row, o_head;
  int32_t batch, seqlen_q, heads_q, num_splits;
};

// Everything the backward kernels need, resolved on the host.  Strides are in
// elements; dsum (D = rowsum(dO * O), fp32) and lse share one indexing:
// b * lse_batch + h * lse_head + (q_start + row).
struct BwdKernelParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* dsum;          // workspace: D, written by the dQ kernel, read by the dK/dV kernel
  void* dq;
  void* dk;
  void* dv;
  const int32_t* cu_seqlens_q;  // varlen prefix sums [B+1] (null: dense)
  const int32_t* cu_seqlens_k;
  int64_t q_batch, q_row, q_head;
  int64_t k_batch, k_row, k_head;
  int64_t v_batch, v_row, v_head;
  int64_t o_batch, o_row, o_head;
  int64_t do_batch, do_row, do_head;
  int64_t dq_batch, dq_row, dq_head;
  int64_t dk_batch, dk_row, dk_head;
  int64_t dv_batch, dv_row, dv_head;
  int64_t lse_batch, lse_head;
  int32_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, group;
  int32_t window_left, window_right;  // causal folded into window_right
  float scale;           // softmax scale (dQ, dK = scale * sum of dS products)
  float scale_log2;      // raw (or capped) score -> exp2 argument, as in the forward
  float softcap_pre;     // scale / softcap
  float softcap;         // 0: off
  float inv_softcap;     // 1 / softcap
  const float* alibi;    // ALiBi slopes (null: off)
  int64_t alibi_bstride;
  float alibi_inv_scale; // bias in the units of the (capped) score
};

constexpr int kBlockM = 128;  // nominal query rows per workgroup (split-count heuristic)

// Compute units of the current device (queried once per device; 256 if the
// query fails).
int compute_units();

// The debug build (-DATTN_DEBUG_BUILD) adds tile-shape overrides for tests
// and sweeps, set through an explicit call, and the per-row rescale
// counters.  The release library has neither: the kernel a call runs
// depends on its arguments alone.
#if defined(ATTN_DEBUG_BUILD) && !defined(ATTN_NO_ROW_STATS)
#define ATTN_ROW_STATS 1  // per-row counters (a sweep build may leave them out)
#endif
#ifdef ATTN_DEBUG_BUILD
constexpr bool kDebugBuild = true;
struct DebugState {
  int fwd_variant;   // forward tile override (0: per-shape default)
  int dec_variant;   // decode tile override
  int bwd_variant;   // backward kernel-shape override
  int last_block_k;  // KV step of the last forward tile launch (process-wide)
};
DebugState& debug_state();
inline int fwd_variant() { return debug_state().fwd_variant; }
inline int dec_variant() { return debug_state().dec_variant; }
inline int bwd_variant() { return debug_state().bwd_variant; }
inline void note_block_k(int bk) { debug_state().last_block_k = bk; }
#else
constexpr bool kDebugBuild = false;
constexpr int fwd_variant() { return 0; }
constexpr int dec_variant() { return 0; }
constexpr int bwd_variant() { return 0; }
inline void note_block_k(int) {}
#endif

// Host-side launchers (return a hipError_t).  Each kernel source is compiled
// once per 16-bit type (ATTN_TU_DTYPE = 0: fp16, 1: bf16); the dispatchers
// below pick the type.
hipError_t launch_fwd_f16(const FwdKernelParams& p, int head_dim, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdKernelParams& p, int head_dim, hipStream_t stream);
hipError_t launch_combine_f16(const CombineParams& p, int head_dim, hipStream_t stream);
hipError_t launch_combine_bf16(const CombineParams& p, int head_dim, hipStream_t stream);
hipError_t launch_bwd_f16(const BwdKernelParams& p, int head_dim, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdKernelParams& p, int head_dim, hipStream_t stream);

inline hipError_t launch_fwd(const FwdKernelParams& p, int dtype, int head_dim, hipStream_t stream) {
  return dtype == 1 ? launch_fwd_bf16(p, head_dim, stream) : launch_fwd_f16(p, head_dim, stream);
}
inline hipError_t launch_combine(const CombineParams& p, int dtype, int head_dim, hipStream_t stream) {
  return dtype == 1 ? launch_combine_bf16(p, head_dim, stream) : launch_combine_f16(p, head_dim, stream);
}
inline hipError_t launch_bwd(const BwdKernelParams& p, int dtype, int head_dim, hipStream_t stream) {
  if (p.batch <= 0 || p.heads_q <= 0) return hipSuccess;
  return dtype == 1 ? launch_bwd_bf16(p, head_dim, stream) : launch_bwd_f16(p, head_dim, stream);
}

}  // namespace attn
