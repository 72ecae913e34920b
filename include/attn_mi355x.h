/*
 * attn_mi355x.h -- C ABI of the exact tiled attention library (forward and
 * backward) for AMD Instinct MI355X (gfx950).
 *
 * The library computes exact attention forward
 *
 *     O = softmax(scale * Q K^T [softcapped] + mask) V,   LSE = ln sum exp(...)
 *
 * in tiles with an online softmax that keeps a running row max and row sum
 * (FlashAttention-2 structure).  The rescale of the running output and sum
 * is skipped whenever the row max rises by no more than `rescale_threshold`
 * in log2 units of the scaled score; on a skip the running max keeps its
 * previous value ("max lagging"), so output, row sum and probabilities stay
 * on one base and the result is exact.  Sources: release page "v1.7 /
 * flash_attn 2.9.2.post1" of the ussoewwin flash-attention fork, section 1.2
 * (threshold 8.0 for 16-bit inputs, lagging, P <= exp2(8) = 256) and
 * section 2 (public features: causal, window, softcap, varlen, kv-cache);
 * release page "FA2 2.9.0 Kernel Changes in v1.2", sections 1-3 (the
 * rescale step, the exp2-domain softmax and its -inf guard, the split-KV
 * kernel).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are device pointers owned by the caller.  The library never
 *    allocates, frees or synchronises; every call only enqueues kernels on
 *    `stream` (a hipStream_t; NULL = the default stream) and returns.
 *  - Q, K, V and O share one 16-bit dtype (ATTN_DTYPE_F16 or _BF16); LSE and
 *    all workspace partials are fp32.
 *  - Strides are in elements (not bytes), int64.  The head dimension is
 *    contiguous (stride 1).  Every pointer must be 16-byte aligned and every
 *    stride a multiple of 8 elements; row strides must be below 2^24.
 *  - head_dim must be 64, 128 or 256.  heads_q must be a multiple of
 *    heads_kv; query head h reads KV head h / (heads_q / heads_kv).
 *  - Masks are aligned to the bottom-right corner: with off = Sk - Sq, key j
 *    is visible to query row i iff (!causal || j <= i + off) and
 *    (window_left < 0 || j >= i + off - window_left) and
 *    (window_right < 0 || j <= i + off + window_right).  -1 means unbounded;
 *    0 is a real (zero-width) bound, so window (0, 0) selects the diagonal.
 *  - softcap > 0 replaces each scaled score t by softcap * tanh(t / softcap)
 *    before masking; 0 disables it.
 *  - softmax_scale <= 0 selects 1/sqrt(head_dim).
 *  - rescale_threshold < 0 selects the default 8.0 (16-bit inputs); 0 gives
 *    the classic always-rescale online softmax.  Any value in [0, 15] gives
 *    the same exact result up to rounding; larger values are rejected
 *    (ATTN_E_ARG), since a skipped rescale lets P reach 2^threshold and P is
 *    rounded to the 16-bit input type (fp16 tops out at 65504).
 *  - LSE is natural-log, fp32.  A query row with no visible key gets O = 0
 *    and LSE = -inf.  `lse` may be NULL.
 *  - Results are deterministic: identical inputs give bit-identical outputs.
 *  - Return value: ATTN_OK (0) or a negative ATTN_E_* code.  All arguments
 *    are validated on the host before anything is enqueued; on error nothing
 *    is launched and outputs are untouched.  An empty problem (no query
 *    rows) returns ATTN_OK and launches nothing.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_VERSION 140

enum attn_status {
  ATTN_OK = 0,
  ATTN_E_NULL = -1,        /* a required pointer is NULL */
  ATTN_E_SHAPE = -2,       /* negative or inconsistent sizes, bad cu_seqlens host hints */
  ATTN_E_HEADS = -3,       /* heads_q % heads_kv != 0 or a head count < 1 */
  ATTN_E_UNSUPPORTED = -4, /* dtype or head_dim not supported */
  ATTN_E_WINDOW = -5,      /* window bound < -1 */
  ATTN_E_WORKSPACE = -6,   /* workspace missing or smaller than required */
  ATTN_E_LAUNCH = -7,      /* the HIP runtime reported an error at launch */
  ATTN_E_ALIGN = -8,       /* pointer or stride alignment / stride range violated */
  ATTN_E_ARG = -9          /* other invalid scalar argument (scale, softcap, splits) */
};

enum attn_dtype { ATTN_DTYPE_F16 = 0, ATTN_DTYPE_BF16 = 1 };

/*
 * Fields shared by the three entry points: features of the softmax.
 * ALiBi (alibi_slopes among the public API features, "v1.7 / flash_attn
 * 2.9.2.post1" section 2 and the API-path table of section 4): when
 * alibi_slopes is not NULL, -slope(b, h) * |i + (Sk - Sq) - j| is added to
 * the final score of query row i and key j (after scale and softcap, before
 * masks and the softmax), with slope(b, h) = alibi_slopes[b *
 * alibi_batch_stride + h], fp32 in device memory, 4-byte aligned
 * (alibi_batch_stride 0: one slope per query head for every batch entry).
 */
typedef struct attn_softmax_opts {
  float softmax_scale;     /* <= 0: 1/sqrt(head_dim) */
  int32_t causal;          /* 0 or 1 */
  int32_t window_left;     /* -1 unbounded, >= 0 bound */
  int32_t window_right;    /* -1 unbounded, >= 0 bound */
  float softcap;           /* 0: off, > 0: tanh cap */
  float rescale_threshold; /* < 0: default 8.0 */
  const float* alibi_slopes;  /* NULL: no ALiBi bias */
  int64_t alibi_batch_stride; /* elements between batch entries of alibi_slopes (>= 0) */
} attn_softmax_opts;

/*
 * attn_fwd -- dense batched attention forward.
 *   q [batch, seqlen_q, heads_q, head_dim]
 *   k, v [batch, seqlen_k, heads_kv, head_dim]
 *   o like q (written), lse [batch, heads_q, seqlen_q] contiguous fp32 (written, may be NULL)
 * Source: "v1.7 / flash_attn 2.9.2.post1" sections 1.2 and 2 (flash_attn_func
 * features); section 4.6 gives the LSE shape [B, H, S].
 */
typedef struct attn_fwd_args {
  int32_t dtype;
  int32_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_batch_stride, q_row_stride, q_head_stride;
  int64_t k_batch_stride, k_row_stride, k_head_stride;
  int64_t v_batch_stride, v_row_stride, v_head_stride;
  int64_t o_batch_stride, o_row_stride, o_head_stride;
  attn_softmax_opts opts;
} attn_fwd_args;

int attn_fwd(const attn_fwd_args* args, void* stream);

/*
 * attn_fwd_varlen -- packed variable-length attention forward
 * (flash_attn_varlen_func in "v1.7 / flash_attn 2.9.2.post1" section 2).
 *   q [total_q, heads_q, head_dim], k, v [total_k, heads_kv, head_dim]
 *   cu_seqlens_q, cu_seqlens_k: device int32 [batch + 1], prefix sums from 0,
 *     non-decreasing; sequence b owns rows cu[b] .. cu[b+1]-1 and attends only
 *     within itself (masks apply per sequence).
 *   max_seqlen_q / max_seqlen_k: host upper bounds of the per-sequence lengths
 *     (used for the grid; a sequence longer than its bound is truncated).
 *   o like q, lse [heads_q, total_q] contiguous fp32 (may be NULL).
 *   workspace: reserved.  attn_varlen_workspace_bytes() is 0 in this version
 *     (the grid is sized by max_seqlen_q and each workgroup reads its
 *     sequence bounds from cu_seqlens on the device; tiles past a sequence's
 *     end exit at once), so workspace may be NULL and is not read.
 */
typedef struct attn_varlen_args {
  int32_t dtype;
  int32_t batch, total_q, total_k, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, head_dim;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int64_t q_row_stride, q_head_stride;
  int64_t k_row_stride, k_head_stride;
  int64_t v_row_stride, v_head_stride;
  int64_t o_row_stride, o_head_stride;
  attn_softmax_opts opts;
} attn_varlen_args;

size_t attn_varlen_workspace_bytes(int32_t batch, int32_t max_seqlen_q, int32_t heads_q,
                                   int32_t heads_kv, int32_t head_dim);
int attn_fwd_varlen(const attn_varlen_args* args, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * attn_fwd_kvcache -- attention of new queries against a KV cache, through
 * the split-KV kernel plus a log-sum-exp combine (flash_attn_with_kvcache in
 * "v1.7 / flash_attn 2.9.2.post1" section 2; the split-KV kernel is the
 * compute_attn_1rowblock_splitkv row of the call-site table in "FA2 2.9.0
 * Kernel Changes in v1.2" section 3).
 *   q [batch, seqlen_q, heads_q, head_dim]
 *   k_cache, v_cache [batch, seqlen_k (capacity), heads_kv, head_dim]
 *   cache_seqlens: device int32 [batch] valid lengths (<= seqlen_k), or NULL
 *     for "all seqlen_k rows valid".  Rows at or past a sequence's valid
 *     length are never read, so they may hold anything (even NaN).
 *   num_splits: number of KV splits (0 = attn_kvcache_num_splits()).
 *   o like q, lse [batch, heads_q, seqlen_q] contiguous fp32 (may be NULL).
 *   workspace: attn_kvcache_workspace_bytes() bytes (fp32 partial outputs and
 *     LSEs of every split); may be NULL when that size is 0 (one split).
 * Paged cache (the paged KV caches of the Python API, "flash-attention"
 * project survey page, csrc/flash_attn entry): when block_table is not NULL,
 *   k_cache, v_cache are [num_pages, page_block_size, heads_kv, head_dim]
 *     (k_batch_stride / v_batch_stride = stride between pages, the row
 *     stride between rows of a page),
 *   block_table: device int32 [batch, block_table_stride]; entry [b, i] is
 *     the page that holds keys i*page_block_size .. (i+1)*page_block_size-1
 *     of sequence b,
 *   page_block_size: a positive multiple of 64 (a KV tile never straddles
 *     pages), seqlen_k <= block_table_stride * page_block_size.
 *   Entries outside [0, num_pages) are clamped into it: no memory outside the
 *   cache is read, but the result is then unspecified.
 *   With block_table NULL the four paging fields are ignored.
 * The result is independent of num_splits up to fp32 rounding, and a paged
 * cache gives the same bits as the contiguous cache it pages.
 */
typedef struct attn_kvcache_args {
  int32_t dtype;
  int32_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim;
  int32_t num_splits;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cache_seqlens;
  void* o;
  float* lse;
  int64_t q_batch_stride, q_row_stride, q_head_stride;
  int64_t k_batch_stride, k_row_stride, k_head_stride;
  int64_t v_batch_stride, v_row_stride, v_head_stride;
  int64_t o_batch_stride, o_row_stride, o_head_stride;
  attn_softmax_opts opts;
  const int32_t* block_table; /* NULL: contiguous cache */
  int32_t block_table_stride;
  int32_t page_block_size;
  int32_t num_pages;
  int32_t reserved0;          /* must be 0 */
} attn_kvcache_args;

/* Split count the library picks when num_splits == 0: about four workgroups
 * per compute unit, at least four 64-key steps per split, at most 128 splits.
 * It is never forced to 1 just because the problem is too small to fill the
 * GPU -- the release notes of fa4-v4.0.0.beta33 on the Dao-AILab
 * "flash-attention" project page report that upstream bug in the ROCm split
 * heuristic.  Returns 1 for empty or non-positive sizes. */
int32_t attn_kvcache_num_splits(int32_t batch, int32_t seqlen_q, int32_t heads_q,
                                int32_t heads_kv, int32_t seqlen_k, int32_t head_dim);
size_t attn_kvcache_workspace_bytes(int32_t batch, int32_t seqlen_q, int32_t heads_q,
                                    int32_t head_dim, int32_t num_splits);
int attn_fwd_kvcache(const attn_kvcache_args* args, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * attn_fwd_kvcache_noalloc -- attn_fwd_kvcache with no workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * allocates nothing (no hipMalloc / hipFree, no allocating library call):
 * the split partials go to a static device array of
 * ATTN_NOALLOC_SCRATCH_BYTES bytes that each GPU holds for the life of the
 * process.  The caller still owns and passes q, the caches, o and lse.
 *   args: as for attn_fwd_kvcache (same validation, same kernels, the same
 *     bits as attn_fwd_kvcache with the same split count).
 *   The scratch of the current device is used, so `stream` must belong to
 *     the current device.
 * Returns ATTN_E_WORKSPACE when attn_kvcache_workspace_bytes() of the call
 * exceeds ATTN_NOALLOC_SCRATCH_BYTES (pick fewer splits), ATTN_E_LAUNCH if
 * the scratch address cannot be obtained, else as attn_fwd_kvcache.
 * Every call on a GPU shares that GPU's scratch: calls that overlap in time
 * on one GPU (different streams without ordering) race and must not be
 * issued; calls on one stream are ordered and safe.  Nothing in the scratch
 * needs to start at zero: every partial the combine reads is written by the
 * same call first.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int attn_fwd_kvcache_noalloc(const attn_kvcache_args* args, void* stream);

/*
 * attn_bwd -- gradients of attn_fwd: dQ, dK, dV for a loss whose gradient
 * with respect to O is dO (the backward kernels the pages list and check
 * against an fp32 reference: "v1.7 / flash_attn 2.9.2.post1" section 4.4).
 * With P recomputed from the scores and the forward's LSE:
 *     dV = P^T dO,  dT = P (dO V^T - D),  D_i = <dO_i, O_i>,
 *     dQ = scale (dT g) K,  dK = scale (dT g)^T Q,
 * g = 1 - (t / softcap)^2 with softcap (t the capped score), else 1; the
 * ALiBi bias adds no term.  Under GQA dK, dV of a KV head sum over its query
 * heads.
 *   q, o, dout [batch, seqlen_q, heads_q, head_dim]
 *   k, v [batch, seqlen_k, heads_kv, head_dim]
 *   lse [batch, heads_q, seqlen_q] contiguous fp32: the LSE attn_fwd returned
 *     for the same inputs and options (a row with LSE = -inf gets dQ = 0 and
 *     adds nothing to dK, dV).
 *   dq like q; dk, dv like k (written, 16-bit).
 *   opts as for attn_fwd; rescale_threshold is not used (the backward does
 *     not run the online softmax).
 *   workspace: attn_bwd_workspace_bytes() bytes (fp32 D per query row).
 *   head_dim 64, 128 or 256 (the project survey page's csrc/flash_attn entry
 *   lists backward kernels up to head dim 256).
 * No atomics: every output element has one owner, so results are
 * deterministic.
 */
typedef struct attn_bwd_args {
  int32_t dtype;
  int32_t batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t q_batch_stride, q_row_stride, q_head_stride;
  int64_t k_batch_stride, k_row_stride, k_head_stride;
  int64_t v_batch_stride, v_row_stride, v_head_stride;
  int64_t o_batch_stride, o_row_stride, o_head_stride;
  int64_t do_batch_stride, do_row_stride, do_head_stride;
  int64_t dq_batch_stride, dq_row_stride, dq_head_stride;
  int64_t dk_batch_stride, dk_row_stride, dk_head_stride;
  int64_t dv_batch_stride, dv_row_stride, dv_head_stride;
  attn_softmax_opts opts;
} attn_bwd_args;

size_t attn_bwd_workspace_bytes(int32_t batch, int32_t seqlen_q, int32_t heads_q);
int attn_bwd(const attn_bwd_args* args, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_varlen -- gradients of attn_fwd_varlen (the pages check the
 * varlen backward for finite gradients, "v1.7 / flash_attn 2.9.2.post1"
 * section 4.4).  Layouts as in attn_fwd_varlen: q, o, dout, dq
 * [total_q, heads_q, head_dim]; k, v, dk, dv [total_k, heads_kv, head_dim];
 * lse [heads_q, total_q] fp32 from attn_fwd_varlen; cu_seqlens_q/_k device
 * int32 [batch + 1]; max_seqlen_q/_k host upper bounds.  workspace:
 * attn_bwd_varlen_workspace_bytes() bytes.
 */
typedef struct attn_bwd_varlen_args {
  int32_t dtype;
  int32_t batch, total_q, total_k, max_seqlen_q, max_seqlen_k, heads_q, heads_kv, head_dim;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int64_t q_row_stride, q_head_stride;
  int64_t k_row_stride, k_head_stride;
  int64_t v_row_stride, v_head_stride;
  int64_t o_row_stride, o_head_stride;
  int64_t do_row_stride, do_head_stride;
  int64_t dq_row_stride, dq_head_stride;
  int64_t dk_row_stride, dk_head_stride;
  int64_t dv_row_stride, dv_head_stride;
  attn_softmax_opts opts;
} attn_bwd_varlen_args;

size_t attn_bwd_varlen_workspace_bytes(int32_t total_q, int32_t heads_q);
int attn_bwd_varlen(const attn_bwd_varlen_args* args, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Human-readable text of a status code (static storage). */
const char* attn_status_string(int status);
/* ATTN_VERSION of the built library. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
