// Host side of the C ABI declared in include/attn_mi355x.h: argument
// validation (pure host code, no HIP call before it succeeds), resolution of
// the softmax options, the split-count heuristic, workspace sizing and the
// kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "attn_internal.h"
#include "attn_mi355x.h"
#ifdef ATTN_DEBUG_BUILD
#include "attn_mi355x_debug.h"
#endif

namespace attn {

// Compute units of the current device (queried once per device; threads that
// race on the first query store the same value).
int compute_units() {
  static std::atomic<int> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int q = 0;
    n = (hipDeviceGetAttribute(&q, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && q > 0) ? q : 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

#ifdef ATTN_DEBUG_BUILD
DebugState& debug_state() {
  static DebugState state = {0, 0, 0, 0};  // process-wide
  return state;
}
#endif

}  // namespace attn

namespace {

using attn::FwdKernelParams;

constexpr int64_t kMaxRowStride = int64_t(1) << 24;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
bool stride_ok(int64_t s) { return s >= 0 && (s & 7) == 0; }
bool row_stride_ok(int64_t s) { return stride_ok(s) && s < kMaxRowStride; }

// A skipped rescale lets P reach 2^threshold; 2^15 still fits fp16 (max 65504).
constexpr float kMaxRescaleThreshold = 15.0f;

int check_common(int32_t dtype, int32_t head_dim, int32_t heads_q, int32_t heads_kv,
                 const attn_softmax_opts& o) {
  if (dtype != ATTN_DTYPE_F16 && dtype != ATTN_DTYPE_BF16) return ATTN_E_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return ATTN_E_UNSUPPORTED;
  if (heads_q < 1 || heads_kv < 1 || heads_q % heads_kv != 0) return ATTN_E_HEADS;
  if (o.window_left < -1 || o.window_right < -1) return ATTN_E_WINDOW;
  if (o.causal != 0 && o.causal != 1) return ATTN_E_ARG;
  if (!std::isfinite(o.softmax_scale) || !std::isfinite(o.softcap) || o.softcap < 0.0f ||
      !std::isfinite(o.rescale_threshold) || o.rescale_threshold > kMaxRescaleThreshold)
    return ATTN_E_ARG;
  if (o.alibi_slopes != nullptr) {
    if (o.alibi_batch_stride < 0) return ATTN_E_ARG;
    if ((reinterpret_cast<uintptr_t>(o.alibi_slopes) & 3u) != 0) return ATTN_E_ALIGN;
  }
  return ATTN_OK;
}

// Fold causal into the right window bound and turn the options into the
// kernel's exp2-domain constants.
void resolve_opts(const attn_softmax_opts& o, int head_dim, FwdKernelParams& p) {
  const float scale = o.softmax_scale > 0.0f ? o.softmax_scale : 1.0f / std::sqrt((float)head_dim);
  const float log2e = 1.4426950408889634f;
  p.window_left = o.window_left;
  p.window_right = o.window_right;
  if (o.causal) p.window_right = 0;  // j <= i + off, tighter than any right bound >= 0
  if (o.softcap > 0.0f) {
    p.softcap = o.softcap;
    p.softcap_pre = scale / o.softcap;
    p.scale_log2 = log2e;
    p.scale_ln = 1.0f;
  } else {
    p.softcap = 0.0f;
    p.softcap_pre = 0.0f;
    p.scale_log2 = scale * log2e;
    p.scale_ln = scale;
  }
  p.tau = o.rescale_threshold < 0.0f ? 8.0f : o.rescale_threshold;
  // ALiBi: the kernel works on raw scores (final score = scale_ln * raw), so
  // it adds the bias divided by scale_ln.
  p.alibi = o.alibi_slopes;
  p.alibi_bstride = o.alibi_batch_stride;
  p.alibi_inv_scale = 1.0f / p.scale_ln;
}

// The backward's constants: the same score units as the forward, plus the
// plain scale (dQ, dK) and 1 / softcap (the softcap derivative).
void resolve_bwd_opts(const attn_softmax_opts& o, int head_dim, attn::BwdKernelParams& p) {
  FwdKernelParams f;
  std::memset(&f, 0, sizeof(f));
  resolve_opts(o, head_dim, f);
  p.window_left = f.window_left;
  p.window_right = f.window_right;
  p.scale = o.softmax_scale > 0.0f ? o.softmax_scale : 1.0f / std::sqrt((float)head_dim);
  p.scale_log2 = f.scale_log2;
  p.softcap_pre = f.softcap_pre;
  p.softcap = f.softcap;
  p.inv_softcap = f.softcap > 0.0f ? 1.0f / f.softcap : 0.0f;
  p.alibi = f.alibi;
  p.alibi_bstride = f.alibi_bstride;
  p.alibi_inv_scale = f.alibi_inv_scale;
}

int launch_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH; }

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_SHAPE: return "invalid or inconsistent sizes";
    case ATTN_E_HEADS: return "heads_q must be a positive multiple of heads_kv";
    case ATTN_E_UNSUPPORTED: return "unsupported dtype or head_dim (64, 128, 256)";
    case ATTN_E_WINDOW: return "window bounds must be >= -1";
    case ATTN_E_WORKSPACE: return "workspace missing or too small";
    case ATTN_E_LAUNCH: return "HIP launch failed";
    case ATTN_E_ALIGN: return "pointers must be 16-byte aligned, strides multiples of 8 elements, row strides < 2^24";
    case ATTN_E_ARG: return "invalid scalar argument";
    default: return "unknown status";
  }
}

int attn_version(void) { return ATTN_VERSION; }

}  // extern "C"

namespace {

// Validation and kernel parameters of attn_fwd.  Returns ATTN_OK with
// `empty` set when there is nothing to launch.
int prepare_fwd(const attn_fwd_args* a, FwdKernelParams& p, bool& empty) {
  empty = false;
  if (a == nullptr) return ATTN_E_NULL;
  int st = check_common(a->dtype, a->head_dim, a->heads_q, a->heads_kv, a->opts);
  if (st != ATTN_OK) return st;
  if (a->batch < 0 || a->seqlen_q < 0 || a->seqlen_k < 0) return ATTN_E_SHAPE;
  if (a->batch == 0 || a->seqlen_q == 0) {  // empty problem: nothing to do
    empty = true;
    return ATTN_OK;
  }
  if (a->q == nullptr || a->o == nullptr) return ATTN_E_NULL;
  if (a->seqlen_k > 0 && (a->k == nullptr || a->v == nullptr)) return ATTN_E_NULL;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o) ||
      !stride_ok(a->q_batch_stride) || !row_stride_ok(a->q_row_stride) || !stride_ok(a->q_head_stride) ||
      !stride_ok(a->k_batch_stride) || !row_stride_ok(a->k_row_stride) || !stride_ok(a->k_head_stride) ||
      !stride_ok(a->v_batch_stride) || !row_stride_ok(a->v_row_stride) || !stride_ok(a->v_head_stride) ||
      !stride_ok(a->o_batch_stride) || !row_stride_ok(a->o_row_stride) || !stride_ok(a->o_head_stride))
    return ATTN_E_ALIGN;
  if (a->lse != nullptr && (reinterpret_cast<uintptr_t>(a->lse) & 3u) != 0) return ATTN_E_ALIGN;

  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.lse = a->lse;
  p.q_batch = a->q_batch_stride; p.q_row = a->q_row_stride; p.q_head = a->q_head_stride;
  p.k_batch = a->k_batch_stride; p.k_row = a->k_row_stride; p.k_head = a->k_head_stride;
  p.v_batch = a->v_batch_stride; p.v_row = a->v_row_stride; p.v_head = a->v_head_stride;
  p.o_batch = a->o_batch_stride; p.o_row = a->o_row_stride; p.o_head = a->o_head_stride;
  p.lse_batch = (int64_t)a->heads_q * a->seqlen_q;
  p.lse_head = a->seqlen_q;
  p.batch = a->batch; p.seqlen_q = a->seqlen_q; p.seqlen_k = a->seqlen_k;
  p.heads_q = a->heads_q; p.heads_kv = a->heads_kv; p.group = a->heads_q / a->heads_kv;
  p.pack_gqa = p.group > 1 ? 1 : 0;
  p.num_splits = 1;
  resolve_opts(a->opts, a->head_dim, p);
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const attn_fwd_args* a, void* stream) {
  FwdKernelParams p;
  bool empty = false;
  const int st = prepare_fwd(a, p, empty);
  if (st != ATTN_OK || empty) return st;
  return launch_status(attn::launch_fwd(p, a->dtype, a->head_dim, (hipStream_t)stream));
}

size_t attn_varlen_workspace_bytes(int32_t, int32_t, int32_t, int32_t, int32_t) { return 0; }

int attn_fwd_varlen(const attn_varlen_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (a == nullptr) return ATTN_E_NULL;
  int st = check_common(a->dtype, a->head_dim, a->heads_q, a->heads_kv, a->opts);
  if (st != ATTN_OK) return st;
  if (a->batch < 0 || a->total_q < 0 || a->total_k < 0 || a->max_seqlen_q < 0 || a->max_seqlen_k < 0)
    return ATTN_E_SHAPE;
  if (a->batch == 0 || a->total_q == 0 || a->max_seqlen_q == 0) return ATTN_OK;
  if (a->q == nullptr || a->o == nullptr || a->cu_seqlens_q == nullptr || a->cu_seqlens_k == nullptr)
    return ATTN_E_NULL;
  if (a->total_k > 0 && (a->k == nullptr || a->v == nullptr)) return ATTN_E_NULL;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o) ||
      !row_stride_ok(a->q_row_stride) || !stride_ok(a->q_head_stride) ||
      !row_stride_ok(a->k_row_stride) || !stride_ok(a->k_head_stride) ||
      !row_stride_ok(a->v_row_stride) || !stride_ok(a->v_head_stride) ||
      !row_stride_ok(a->o_row_stride) || !stride_ok(a->o_head_stride))
    return ATTN_E_ALIGN;
  if (a->lse != nullptr && (reinterpret_cast<uintptr_t>(a->lse) & 3u) != 0) return ATTN_E_ALIGN;

  FwdKernelParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.lse = a->lse;
  p.cu_seqlens_q = a->cu_seqlens_q; p.cu_seqlens_k = a->cu_seqlens_k;
  p.q_row = a->q_row_stride; p.q_head = a->q_head_stride;
  p.k_row = a->k_row_stride; p.k_head = a->k_head_stride;
  p.v_row = a->v_row_stride; p.v_head = a->v_head_stride;
  p.o_row = a->o_row_stride; p.o_head = a->o_head_stride;
  p.lse_batch = 0;
  p.lse_head = a->total_q;
  p.batch = a->batch; p.seqlen_q = a->max_seqlen_q; p.seqlen_k = a->max_seqlen_k;
  p.heads_q = a->heads_q; p.heads_kv = a->heads_kv; p.group = a->heads_q / a->heads_kv;
  p.pack_gqa = p.group > 1 ? 1 : 0;
  p.num_splits = 1;
  resolve_opts(a->opts, a->head_dim, p);
  return launch_status(attn::launch_fwd(p, a->dtype, a->head_dim, (hipStream_t)stream));
}

int32_t attn_kvcache_num_splits(int32_t batch, int32_t seqlen_q, int32_t heads_q, int32_t heads_kv,
                                int32_t seqlen_k, int32_t head_dim) {
  (void)head_dim;
  if (batch <= 0 || seqlen_q <= 0 || heads_q <= 0 || heads_kv <= 0 || seqlen_k <= 0) return 1;
  const int64_t group = heads_q / heads_kv;
  const int64_t m_tiles = ((int64_t)seqlen_q * group + attn::kBlockM - 1) / attn::kBlockM;
  const int64_t base = (int64_t)batch * heads_kv * m_tiles;  // workgroups without splitting
  const int64_t target = 4 * 256;                           // ~4 workgroups per compute unit
  const int64_t kv_steps = (seqlen_k + 63) / 64;
  int64_t s = (target + base - 1) / base;
  s = std::min<int64_t>(s, std::max<int64_t>(1, kv_steps / 4));  // keep >= 4 KV steps per split
  s = std::max<int64_t>(1, std::min<int64_t>(s, 128));
  return (int32_t)s;
}

size_t attn_kvcache_workspace_bytes(int32_t batch, int32_t seqlen_q, int32_t heads_q, int32_t head_dim,
                                    int32_t num_splits) {
  if (num_splits <= 1 || batch <= 0 || seqlen_q <= 0 || heads_q <= 0 || head_dim <= 0) return 0;
  const size_t rows = (size_t)num_splits * batch * heads_q * seqlen_q;
  return rows * (size_t)head_dim * sizeof(float) + rows * sizeof(float);
}

}  // extern "C"

namespace {

// Validation and kernel parameters of attn_fwd_kvcache, everything but the
// workspace.  Returns ATTN_OK with `empty` set when there is nothing to
// launch; `need` is the workspace the call requires.
int prepare_kvcache(const attn_kvcache_args* a, FwdKernelParams& p, size_t& need, bool& empty) {
  empty = false;
  need = 0;
  if (a == nullptr) return ATTN_E_NULL;
  int st = check_common(a->dtype, a->head_dim, a->heads_q, a->heads_kv, a->opts);
  if (st != ATTN_OK) return st;
  if (a->batch < 0 || a->seqlen_q < 0 || a->seqlen_k < 0) return ATTN_E_SHAPE;
  if (a->num_splits < 0 || a->num_splits > 256) return ATTN_E_ARG;
  if (a->batch == 0 || a->seqlen_q == 0) {
    empty = true;
    return ATTN_OK;
  }
  if (a->q == nullptr || a->o == nullptr) return ATTN_E_NULL;
  if (a->seqlen_k > 0 && (a->k_cache == nullptr || a->v_cache == nullptr)) return ATTN_E_NULL;
  if (a->block_table != nullptr) {
    if (a->reserved0 != 0 || a->page_block_size <= 0 || a->page_block_size % 64 != 0) return ATTN_E_ARG;
    if (a->num_pages <= 0 || a->block_table_stride <= 0 ||
        (int64_t)a->block_table_stride * a->page_block_size < a->seqlen_k)
      return ATTN_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(a->block_table) & 3u) != 0) return ATTN_E_ALIGN;
  }
  if (!aligned16(a->q) || !aligned16(a->k_cache) || !aligned16(a->v_cache) || !aligned16(a->o) ||
      !stride_ok(a->q_batch_stride) || !row_stride_ok(a->q_row_stride) || !stride_ok(a->q_head_stride) ||
      !stride_ok(a->k_batch_stride) || !row_stride_ok(a->k_row_stride) || !stride_ok(a->k_head_stride) ||
      !stride_ok(a->v_batch_stride) || !row_stride_ok(a->v_row_stride) || !stride_ok(a->v_head_stride) ||
      !stride_ok(a->o_batch_stride) || !row_stride_ok(a->o_row_stride) || !stride_ok(a->o_head_stride))
    return ATTN_E_ALIGN;
  if (a->lse != nullptr && (reinterpret_cast<uintptr_t>(a->lse) & 3u) != 0) return ATTN_E_ALIGN;
  const int32_t splits = a->num_splits > 0
                             ? a->num_splits
                             : attn_kvcache_num_splits(a->batch, a->seqlen_q, a->heads_q, a->heads_kv,
                                                       a->seqlen_k, a->head_dim);
  need = attn_kvcache_workspace_bytes(a->batch, a->seqlen_q, a->heads_q, a->head_dim, splits);

  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.k = a->k_cache; p.v = a->v_cache; p.o = a->o; p.lse = a->lse;
  p.seqused_k = a->cache_seqlens;
  if (a->block_table != nullptr) {
    p.block_table = a->block_table;
    p.bt_stride = a->block_table_stride;
    p.page_size = a->page_block_size;
    p.num_pages = a->num_pages;
  }
  p.q_batch = a->q_batch_stride; p.q_row = a->q_row_stride; p.q_head = a->q_head_stride;
  p.k_batch = a->k_batch_stride; p.k_row = a->k_row_stride; p.k_head = a->k_head_stride;
  p.v_batch = a->v_batch_stride; p.v_row = a->v_row_stride; p.v_head = a->v_head_stride;
  p.o_batch = a->o_batch_stride; p.o_row = a->o_row_stride; p.o_head = a->o_head_stride;
  p.lse_batch = (int64_t)a->heads_q * a->seqlen_q;
  p.lse_head = a->seqlen_q;
  p.batch = a->batch; p.seqlen_q = a->seqlen_q; p.seqlen_k = a->seqlen_k;
  p.heads_q = a->heads_q; p.heads_kv = a->heads_kv; p.group = a->heads_q / a->heads_kv;
  p.pack_gqa = p.group > 1 ? 1 : 0;
  p.num_splits = splits;
  resolve_opts(a->opts, a->head_dim, p);
  return ATTN_OK;
}

// Device scratch of attn_fwd_kvcache_noalloc: the fp32 split partials live
// here instead of in a caller workspace.  Every GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` names only a
// host-side stand-in, so kernels are given the device address that
// hipGetSymbolAddress returns for it, fetched once per device with that
// device current and kept in scratch_ptr.
static __device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

std::mutex scratch_mu;
void* scratch_ptr[64] = {nullptr};

// Device address of the current device's scratch (nullptr on failure).
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}

// Split kernel (fp32 partials in `workspace` when there is more than one
// split) and the combine, on the caller's stream.
int launch_kvcache(const attn_kvcache_args* a, FwdKernelParams& p, void* workspace, hipStream_t stream) {
  const int32_t splits = p.num_splits;
  if (splits > 1) {
    const size_t rows = (size_t)splits * a->batch * a->heads_q * a->seqlen_q;
    p.o_part = static_cast<float*>(workspace);
    p.lse_part = p.o_part + rows * a->head_dim;
  }
  hipError_t e = attn::launch_fwd(p, a->dtype, a->head_dim, stream);
  if (e != hipSuccess || splits == 1) return launch_status(e);
  attn::CombineParams c;
  c.o_part = p.o_part; c.lse_part = p.lse_part; c.o = a->o; c.lse = a->lse;
  c.o_batch = a->o_batch_stride; c.o_row = a->o_row_stride; c.o_head = a->o_head_stride;
  c.batch = a->batch; c.seqlen_q = a->seqlen_q; c.heads_q = a->heads_q; c.num_splits = splits;
  return launch_status(attn::launch_combine(c, a->dtype, a->head_dim, stream));
}

}  // namespace

extern "C" {

int attn_fwd_kvcache(const attn_kvcache_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  FwdKernelParams p;
  size_t need = 0;
  bool empty = false;
  const int st = prepare_kvcache(a, p, need, empty);
  if (st != ATTN_OK || empty) return st;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return ATTN_E_WORKSPACE;
  return launch_kvcache(a, p, workspace, (hipStream_t)stream);
}

int attn_fwd_kvcache_noalloc(const attn_kvcache_args* a, void* stream) {
  FwdKernelParams p;
  size_t need = 0;
  bool empty = false;
  const int st = prepare_kvcache(a, p, need, empty);
  if (st != ATTN_OK || empty) return st;
  if (need > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_E_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_of_current_device();
    if (ws == nullptr) return ATTN_E_LAUNCH;
  }
  return launch_kvcache(a, p, ws, (hipStream_t)stream);
}

size_t attn_bwd_workspace_bytes(int32_t batch, int32_t seqlen_q, int32_t heads_q) {
  if (batch <= 0 || seqlen_q <= 0 || heads_q <= 0) return 0;
  return (size_t)batch * heads_q * seqlen_q * sizeof(float);
}

int attn_bwd(const attn_bwd_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  if (a == nullptr) return ATTN_E_NULL;
  int st = check_common(a->dtype, a->head_dim, a->heads_q, a->heads_kv, a->opts);
  if (st != ATTN_OK) return st;
  if (a->batch < 0 || a->seqlen_q < 0 || a->seqlen_k < 0) return ATTN_E_SHAPE;
  if (a->batch == 0 || (a->seqlen_q == 0 && a->seqlen_k == 0)) return ATTN_OK;
  if (a->seqlen_q > 0 && (a->q == nullptr || a->o == nullptr || a->dout == nullptr || a->lse == nullptr ||
                          a->dq == nullptr))
    return ATTN_E_NULL;
  if (a->seqlen_k > 0 && (a->k == nullptr || a->v == nullptr || a->dk == nullptr || a->dv == nullptr))
    return ATTN_E_NULL;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o) || !aligned16(a->dout) ||
      !aligned16(a->dq) || !aligned16(a->dk) || !aligned16(a->dv) ||
      !stride_ok(a->q_batch_stride) || !row_stride_ok(a->q_row_stride) || !stride_ok(a->q_head_stride) ||
      !stride_ok(a->k_batch_stride) || !row_stride_ok(a->k_row_stride) || !stride_ok(a->k_head_stride) ||
      !stride_ok(a->v_batch_stride) || !row_stride_ok(a->v_row_stride) || !stride_ok(a->v_head_stride) ||
      !stride_ok(a->o_batch_stride) || !row_stride_ok(a->o_row_stride) || !stride_ok(a->o_head_stride) ||
      !stride_ok(a->do_batch_stride) || !row_stride_ok(a->do_row_stride) || !stride_ok(a->do_head_stride) ||
      !stride_ok(a->dq_batch_stride) || !row_stride_ok(a->dq_row_stride) || !stride_ok(a->dq_head_stride) ||
      !stride_ok(a->dk_batch_stride) || !row_stride_ok(a->dk_row_stride) || !stride_ok(a->dk_head_stride) ||
      !stride_ok(a->dv_batch_stride) || !row_stride_ok(a->dv_row_stride) || !stride_ok(a->dv_head_stride))
    return ATTN_E_ALIGN;
  if ((reinterpret_cast<uintptr_t>(a->lse) & 3u) != 0) return ATTN_E_ALIGN;
  const size_t need = attn_bwd_workspace_bytes(a->batch, a->seqlen_q, a->heads_q);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return ATTN_E_WORKSPACE;

  attn::BwdKernelParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.dout = a->dout; p.lse = a->lse;
  p.dsum = static_cast<float*>(workspace);
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
  p.q_batch = a->q_batch_stride; p.q_row = a->q_row_stride; p.q_head = a->q_head_stride;
  p.k_batch = a->k_batch_stride; p.k_row = a->k_row_stride; p.k_head = a->k_head_stride;
  p.v_batch = a->v_batch_stride; p.v_row = a->v_row_stride; p.v_head = a->v_head_stride;
  p.o_batch = a->o_batch_stride; p.o_row = a->o_row_stride; p.o_head = a->o_head_stride;
  p.do_batch = a->do_batch_stride; p.do_row = a->do_row_stride; p.do_head = a->do_head_stride;
  p.dq_batch = a->dq_batch_stride; p.dq_row = a->dq_row_stride; p.dq_head = a->dq_head_stride;
  p.dk_batch = a->dk_batch_stride; p.dk_row = a->dk_row_stride; p.dk_head = a->dk_head_stride;
  p.dv_batch = a->dv_batch_stride; p.dv_row = a->dv_row_stride; p.dv_head = a->dv_head_stride;
  p.lse_batch = (int64_t)a->heads_q * a->seqlen_q;
  p.lse_head = a->seqlen_q;
  p.batch = a->batch; p.seqlen_q = a->seqlen_q; p.seqlen_k = a->seqlen_k;
  p.heads_q = a->heads_q; p.heads_kv = a->heads_kv; p.group = a->heads_q / a->heads_kv;
  if ((int64_t)a->batch * a->seqlen_q > INT32_MAX) return ATTN_E_SHAPE;
  resolve_bwd_opts(a->opts, a->head_dim, p);
  return launch_status(attn::launch_bwd(p, a->dtype, a->head_dim, (hipStream_t)stream));
}

size_t attn_bwd_varlen_workspace_bytes(int32_t total_q, int32_t heads_q) {
  if (total_q <= 0 || heads_q <= 0) return 0;
  return (size_t)total_q * heads_q * sizeof(float);
}

int attn_bwd_varlen(const attn_bwd_varlen_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  if (a == nullptr) return ATTN_E_NULL;
  int st = check_common(a->dtype, a->head_dim, a->heads_q, a->heads_kv, a->opts);
  if (st != ATTN_OK) return st;
  if (a->batch < 0 || a->total_q < 0 || a->total_k < 0 || a->max_seqlen_q < 0 || a->max_seqlen_k < 0)
    return ATTN_E_SHAPE;
  if (a->batch == 0 || (a->total_q == 0 && a->total_k == 0)) return ATTN_OK;
  if (a->cu_seqlens_q == nullptr || a->cu_seqlens_k == nullptr) return ATTN_E_NULL;
  if (a->total_q > 0 && (a->q == nullptr || a->o == nullptr || a->dout == nullptr || a->lse == nullptr ||
                         a->dq == nullptr))
    return ATTN_E_NULL;
  if (a->total_k > 0 && (a->k == nullptr || a->v == nullptr || a->dk == nullptr || a->dv == nullptr))
    return ATTN_E_NULL;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o) || !aligned16(a->dout) ||
      !aligned16(a->dq) || !aligned16(a->dk) || !aligned16(a->dv) ||
      !row_stride_ok(a->q_row_stride) || !stride_ok(a->q_head_stride) ||
      !row_stride_ok(a->k_row_stride) || !stride_ok(a->k_head_stride) ||
      !row_stride_ok(a->v_row_stride) || !stride_ok(a->v_head_stride) ||
      !row_stride_ok(a->o_row_stride) || !stride_ok(a->o_head_stride) ||
      !row_stride_ok(a->do_row_stride) || !stride_ok(a->do_head_stride) ||
      !row_stride_ok(a->dq_row_stride) || !stride_ok(a->dq_head_stride) ||
      !row_stride_ok(a->dk_row_stride) || !stride_ok(a->dk_head_stride) ||
      !row_stride_ok(a->dv_row_stride) || !stride_ok(a->dv_head_stride))
    return ATTN_E_ALIGN;
  if ((reinterpret_cast<uintptr_t>(a->lse) & 3u) != 0) return ATTN_E_ALIGN;
  const size_t need = attn_bwd_varlen_workspace_bytes(a->total_q, a->heads_q);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return ATTN_E_WORKSPACE;

  attn::BwdKernelParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o; p.dout = a->dout; p.lse = a->lse;
  p.dsum = static_cast<float*>(workspace);
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
  p.cu_seqlens_q = a->cu_seqlens_q; p.cu_seqlens_k = a->cu_seqlens_k;
  p.q_row = a->q_row_stride; p.q_head = a->q_head_stride;
  p.k_row = a->k_row_stride; p.k_head = a->k_head_stride;
  p.v_row = a->v_row_stride; p.v_head = a->v_head_stride;
  p.o_row = a->o_row_stride; p.o_head = a->o_head_stride;
  p.do_row = a->do_row_stride; p.do_head = a->do_head_stride;
  p.dq_row = a->dq_row_stride; p.dq_head = a->dq_head_stride;
  p.dk_row = a->dk_row_stride; p.dk_head = a->dk_head_stride;
  p.dv_row = a->dv_row_stride; p.dv_head = a->dv_head_stride;
  p.lse_batch = 0;
  p.lse_head = a->total_q;
  p.batch = a->batch; p.seqlen_q = a->max_seqlen_q; p.seqlen_k = a->max_seqlen_k;
  p.heads_q = a->heads_q; p.heads_kv = a->heads_kv; p.group = a->heads_q / a->heads_kv;
  resolve_bwd_opts(a->opts, a->head_dim, p);
  return launch_status(attn::launch_bwd(p, a->dtype, a->head_dim, (hipStream_t)stream));
}

#ifdef ATTN_DEBUG_BUILD
void attn_debug_set_variants(int32_t fwd, int32_t dec, int32_t bwd) {
  attn::DebugState& d = attn::debug_state();
  d.fwd_variant = fwd;
  d.dec_variant = dec;
  d.bwd_variant = bwd;
}

int32_t attn_debug_last_block_k(void) { return attn::debug_state().last_block_k; }

int attn_fwd_stats(const attn_fwd_args* a, uint32_t* row_stats, void* stream) {
  FwdKernelParams p;
  bool empty = false;
  const int st = prepare_fwd(a, p, empty);
  if (st != ATTN_OK || empty) return st;
#ifndef ATTN_ROW_STATS
  return ATTN_E_UNSUPPORTED;  // a sweep build without the counters
#endif
  if (row_stats == nullptr) return ATTN_E_NULL;
  if (!aligned16(row_stats)) return ATTN_E_ALIGN;
  p.row_stats = row_stats;
  return launch_status(attn::launch_fwd(p, a->dtype, a->head_dim, (hipStream_t)stream));
}
#endif

}  // extern "C"
