"""ctypes binding of libattn_mi355x.so (argument marshalling only).

Every function here maps torch tensors to pointers, strides and the current
HIP stream and calls the C entry point of the same name; all computation
happens in the HIP kernels.  There is no fallback: if the library is not
built, loading fails with an error that says how to build it.
"""

import ctypes
import os

import torch

from .build_lib import LIB_PATH

ATTN_OK = 0
ATTN_E_NULL = -1
ATTN_E_SHAPE = -2
ATTN_E_HEADS = -3
ATTN_E_UNSUPPORTED = -4
ATTN_E_WINDOW = -5
ATTN_E_WORKSPACE = -6
ATTN_E_LAUNCH = -7
ATTN_E_ALIGN = -8
ATTN_E_ARG = -9

ATTN_DTYPE_F16 = 0
ATTN_DTYPE_BF16 = 1
_DTYPE_CODES = {torch.float16: ATTN_DTYPE_F16, torch.bfloat16: ATTN_DTYPE_BF16}

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_vp = ctypes.c_void_p


class SoftmaxOpts(ctypes.Structure):
    _fields_ = [("softmax_scale", _f32), ("causal", _i32), ("window_left", _i32),
                ("window_right", _i32), ("softcap", _f32), ("rescale_threshold", _f32),
                ("alibi_slopes", _vp), ("alibi_batch_stride", _i64)]


class FwdArgs(ctypes.Structure):
    _fields_ = [("dtype", _i32), ("batch", _i32), ("seqlen_q", _i32), ("seqlen_k", _i32),
                ("heads_q", _i32), ("heads_kv", _i32), ("head_dim", _i32),
                ("q", _vp), ("k", _vp), ("v", _vp), ("o", _vp), ("lse", _vp),
                ("q_batch_stride", _i64), ("q_row_stride", _i64), ("q_head_stride", _i64),
                ("k_batch_stride", _i64), ("k_row_stride", _i64), ("k_head_stride", _i64),
                ("v_batch_stride", _i64), ("v_row_stride", _i64), ("v_head_stride", _i64),
                ("o_batch_stride", _i64), ("o_row_stride", _i64), ("o_head_stride", _i64),
                ("opts", SoftmaxOpts)]


class VarlenArgs(ctypes.Structure):
    _fields_ = [("dtype", _i32), ("batch", _i32), ("total_q", _i32), ("total_k", _i32),
                ("max_seqlen_q", _i32), ("max_seqlen_k", _i32), ("heads_q", _i32),
                ("heads_kv", _i32), ("head_dim", _i32),
                ("q", _vp), ("k", _vp), ("v", _vp), ("o", _vp), ("lse", _vp),
                ("cu_seqlens_q", _vp), ("cu_seqlens_k", _vp),
                ("q_row_stride", _i64), ("q_head_stride", _i64),
                ("k_row_stride", _i64), ("k_head_stride", _i64),
                ("v_row_stride", _i64), ("v_head_stride", _i64),
                ("o_row_stride", _i64), ("o_head_stride", _i64),
                ("opts", SoftmaxOpts)]


class KvcacheArgs(ctypes.Structure):
    _fields_ = [("dtype", _i32), ("batch", _i32), ("seqlen_q", _i32), ("seqlen_k", _i32),
                ("heads_q", _i32), ("heads_kv", _i32), ("head_dim", _i32), ("num_splits", _i32),
                ("q", _vp), ("k_cache", _vp), ("v_cache", _vp), ("cache_seqlens", _vp),
                ("o", _vp), ("lse", _vp),
                ("q_batch_stride", _i64), ("q_row_stride", _i64), ("q_head_stride", _i64),
                ("k_batch_stride", _i64), ("k_row_stride", _i64), ("k_head_stride", _i64),
                ("v_batch_stride", _i64), ("v_row_stride", _i64), ("v_head_stride", _i64),
                ("o_batch_stride", _i64), ("o_row_stride", _i64), ("o_head_stride", _i64),
                ("opts", SoftmaxOpts),
                ("block_table", _vp), ("block_table_stride", _i32), ("page_block_size", _i32),
                ("num_pages", _i32), ("reserved0", _i32)]


_STRIDES3 = [f"{t}_{k}_stride" for t in ("q", "k", "v", "o", "do", "dq", "dk", "dv")
             for k in ("batch", "row", "head")]
_STRIDES2 = [f"{t}_{k}_stride" for t in ("q", "k", "v", "o", "do", "dq", "dk", "dv")
             for k in ("row", "head")]


class BwdArgs(ctypes.Structure):
    _fields_ = [("dtype", _i32), ("batch", _i32), ("seqlen_q", _i32), ("seqlen_k", _i32),
                ("heads_q", _i32), ("heads_kv", _i32), ("head_dim", _i32),
                ("q", _vp), ("k", _vp), ("v", _vp), ("o", _vp), ("dout", _vp), ("lse", _vp),
                ("dq", _vp), ("dk", _vp), ("dv", _vp)] + \
               [(n, _i64) for n in _STRIDES3] + [("opts", SoftmaxOpts)]


class BwdVarlenArgs(ctypes.Structure):
    _fields_ = [("dtype", _i32), ("batch", _i32), ("total_q", _i32), ("total_k", _i32),
                ("max_seqlen_q", _i32), ("max_seqlen_k", _i32), ("heads_q", _i32),
                ("heads_kv", _i32), ("head_dim", _i32),
                ("q", _vp), ("k", _vp), ("v", _vp), ("o", _vp), ("dout", _vp), ("lse", _vp),
                ("dq", _vp), ("dk", _vp), ("dv", _vp), ("cu_seqlens_q", _vp), ("cu_seqlens_k", _vp)] + \
               [(n, _i64) for n in _STRIDES2] + [("opts", SoftmaxOpts)]


_LIB = None
_OVERRIDE = []  # libraries pushed by exact_tiled_attention_fa2_amd.debug (tests and sweeps only)


def configure(h):
    """Declare the argument and return types of every entry point of attn_mi355x.h on handle h."""
    h.attn_fwd.argtypes = [ctypes.POINTER(FwdArgs), _vp]
    h.attn_fwd.restype = ctypes.c_int
    h.attn_fwd_varlen.argtypes = [ctypes.POINTER(VarlenArgs), _vp, ctypes.c_size_t, _vp]
    h.attn_fwd_varlen.restype = ctypes.c_int
    h.attn_fwd_kvcache.argtypes = [ctypes.POINTER(KvcacheArgs), _vp, ctypes.c_size_t, _vp]
    h.attn_fwd_kvcache.restype = ctypes.c_int
    h.attn_fwd_kvcache_noalloc.argtypes = [ctypes.POINTER(KvcacheArgs), _vp]
    h.attn_fwd_kvcache_noalloc.restype = ctypes.c_int
    h.attn_varlen_workspace_bytes.argtypes = [_i32] * 5
    h.attn_varlen_workspace_bytes.restype = ctypes.c_size_t
    h.attn_kvcache_workspace_bytes.argtypes = [_i32] * 5
    h.attn_kvcache_workspace_bytes.restype = ctypes.c_size_t
    h.attn_kvcache_num_splits.argtypes = [_i32] * 6
    h.attn_kvcache_num_splits.restype = _i32
    h.attn_bwd.argtypes = [ctypes.POINTER(BwdArgs), _vp, ctypes.c_size_t, _vp]
    h.attn_bwd.restype = ctypes.c_int
    h.attn_bwd_workspace_bytes.argtypes = [_i32] * 3
    h.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    h.attn_bwd_varlen.argtypes = [ctypes.POINTER(BwdVarlenArgs), _vp, ctypes.c_size_t, _vp]
    h.attn_bwd_varlen.restype = ctypes.c_int
    h.attn_bwd_varlen_workspace_bytes.argtypes = [_i32] * 2
    h.attn_bwd_varlen_workspace_bytes.restype = ctypes.c_size_t
    h.attn_status_string.argtypes = [ctypes.c_int]
    h.attn_status_string.restype = ctypes.c_char_p
    h.attn_version.argtypes = []
    h.attn_version.restype = ctypes.c_int
    return h


def lib():
    """The library the entry points below call: the release build (raises if it is not
    built), or the debug build while a test holds exact_tiled_attention_fa2_amd.debug's
    override."""
    global _LIB
    if _OVERRIDE:
        return _OVERRIDE[-1]
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m exact_tiled_attention_fa2_amd.build_lib`")
        _LIB = configure(ctypes.CDLL(LIB_PATH))
    return _LIB


def status_string(code):
    return lib().attn_status_string(int(code)).decode()


def _check(code, what):
    if code != ATTN_OK:
        raise RuntimeError(f"{what} failed: {status_string(code)} (status {code})")


def _opts(causal, window, softcap, softmax_scale, rescale_threshold, alibi_slopes=None):
    """The options struct; alibi_slopes: fp32 GPU tensor [Hq] or [B, Hq] (rows contiguous)."""
    stride = 0
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or alibi_slopes.dim() not in (1, 2) \
                or alibi_slopes.stride(-1) != 1:
            raise TypeError("alibi_slopes must be a float32 [heads_q] or [batch, heads_q] tensor "
                            "with contiguous rows")
        _need_gpu(alibi_slopes)
        stride = alibi_slopes.stride(0) if alibi_slopes.dim() == 2 else 0
    return SoftmaxOpts(float(softmax_scale) if softmax_scale is not None else 0.0, int(bool(causal)),
                       int(window[0]), int(window[1]), float(softcap), float(rescale_threshold),
                       _ptr(alibi_slopes), stride)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    if t.dtype not in _DTYPE_CODES:
        raise TypeError(f"unsupported dtype {t.dtype}; use float16 or bfloat16")
    return _DTYPE_CODES[t.dtype]


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def attn_fwd(q, k, v, causal=False, window=(-1, -1), softcap=0.0, softmax_scale=None,
             rescale_threshold=-1.0, out=None, lse=None, return_lse=True, stream=None,
             alibi_slopes=None):
    """Dense attention forward: q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D] -> (o, lse [B, Hq, Sq])."""
    _need_gpu(q, k, v)
    b, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None and return_lse:
        lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    a = FwdArgs(_dtype_code(q), b, sq, sk, hq, hkv, d, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                *q.stride()[:3], *k.stride()[:3], *v.stride()[:3], *out.stride()[:3],
                _opts(causal, window, softcap, softmax_scale, rescale_threshold, alibi_slopes))
    if q.stride(3) != 1 or k.stride(3) != 1 or v.stride(3) != 1 or out.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    if k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise TypeError("q, k, v and out must share one dtype")
    _check(lib().attn_fwd(ctypes.byref(a), _stream(stream, q.device)), "attn_fwd")
    return out, lse


def attn_varlen_workspace_bytes(batch, max_seqlen_q, heads_q, heads_kv, head_dim):
    return int(lib().attn_varlen_workspace_bytes(batch, max_seqlen_q, heads_q, heads_kv, head_dim))


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal=False,
                    window=(-1, -1), softcap=0.0, softmax_scale=None, rescale_threshold=-1.0,
                    out=None, lse=None, return_lse=True, workspace=None, stream=None,
                    alibi_slopes=None):
    """Packed varlen forward: q [Tq, Hq, D], k/v [Tk, Hkv, D] -> (o, lse [Hq, Tq])."""
    _need_gpu(q, k, v, cu_seqlens_q, cu_seqlens_k)
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    batch = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    need = attn_varlen_workspace_bytes(batch, max_seqlen_q, hq, hkv, d)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    a = VarlenArgs(_dtype_code(q), batch, tq, tk, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d,
                   _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                   _ptr(cu_seqlens_k), *q.stride()[:2], *k.stride()[:2], *v.stride()[:2],
                   *out.stride()[:2], _opts(causal, window, softcap, softmax_scale, rescale_threshold,
                                              alibi_slopes))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().attn_fwd_varlen(ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(stream, q.device)),
           "attn_fwd_varlen")
    return out, lse


def attn_kvcache_num_splits(batch, seqlen_q, heads_q, heads_kv, seqlen_k, head_dim):
    return int(lib().attn_kvcache_num_splits(batch, seqlen_q, heads_q, heads_kv, seqlen_k, head_dim))


def attn_kvcache_workspace_bytes(batch, seqlen_q, heads_q, head_dim, num_splits):
    return int(lib().attn_kvcache_workspace_bytes(batch, seqlen_q, heads_q, head_dim, num_splits))


def _kvcache_args(q, k_cache, v_cache, cache_seqlens, num_splits, causal, window, softcap, softmax_scale,
                  rescale_threshold, out, lse, block_table, alibi_slopes):
    """The attn_kvcache_args struct of one call (num_splits passed through: 0 = the library's pick)."""
    b, sq, hq, d = q.shape
    hkv = k_cache.shape[2]
    if block_table is None:
        sk = k_cache.shape[1]
        paging = (None, 0, 0, 0)
    else:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
            raise TypeError("block_table must be an int32 [batch, pages] tensor with contiguous rows")
        page = k_cache.shape[1]
        sk = block_table.shape[1] * page
        paging = (block_table, block_table.stride(0), page, k_cache.shape[0])
    if cache_seqlens is not None and cache_seqlens.dtype != torch.int32:
        raise TypeError("cache_seqlens must be int32")
    return KvcacheArgs(_dtype_code(q), b, sq, sk, hq, hkv, d, int(num_splits), _ptr(q), _ptr(k_cache),
                       _ptr(v_cache), _ptr(cache_seqlens), _ptr(out), _ptr(lse),
                       *q.stride()[:3], *k_cache.stride()[:3], *v_cache.stride()[:3], *out.stride()[:3],
                       _opts(causal, window, softcap, softmax_scale, rescale_threshold, alibi_slopes),
                       _ptr(paging[0]), paging[1], paging[2], paging[3], 0)


def attn_fwd_kvcache(q, k_cache, v_cache, cache_seqlens=None, num_splits=0, causal=False,
                     window=(-1, -1), softcap=0.0, softmax_scale=None, rescale_threshold=-1.0,
                     out=None, lse=None, return_lse=True, workspace=None, stream=None,
                     block_table=None, alibi_slopes=None):
    """Split-KV attention against a cache: q [B, Sq, Hq, D], caches [B, Sk, Hkv, D].

    Paged cache: with block_table (int32 [B, max_pages_per_seq]) the caches are
    [num_pages, page_block_size, Hkv, D] and the capacity per sequence is
    max_pages_per_seq * page_block_size.
    """
    _need_gpu(q, k_cache, v_cache, cache_seqlens, block_table)
    b, sq, hq, d = q.shape
    hkv = k_cache.shape[2]
    sk = k_cache.shape[1] if block_table is None else block_table.shape[1] * k_cache.shape[1]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None and return_lse:
        lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    splits = int(num_splits) if num_splits else attn_kvcache_num_splits(b, sq, hq, hkv, sk, d)
    need = attn_kvcache_workspace_bytes(b, sq, hq, d, splits)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    a = _kvcache_args(q, k_cache, v_cache, cache_seqlens, splits, causal, window, softcap, softmax_scale,
                      rescale_threshold, out, lse, block_table, alibi_slopes)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().attn_fwd_kvcache(ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(stream, q.device)),
           "attn_fwd_kvcache")
    return out, lse


def attn_fwd_kvcache_noalloc(q, k_cache, v_cache, out, lse=None, cache_seqlens=None, num_splits=0,
                             causal=False, window=(-1, -1), softcap=0.0, softmax_scale=None,
                             rescale_threshold=-1.0, stream=None, block_table=None, alibi_slopes=None):
    """attn_fwd_kvcache through the entry point that allocates nothing: the caller passes the
    output (and optionally the LSE) tensor, and the split partials live in the library's static
    per-GPU scratch (at most ATTN_NOALLOC_SCRATCH_BYTES).  Nothing here allocates either."""
    _need_gpu(q, k_cache, v_cache, out, lse, cache_seqlens, block_table)
    a = _kvcache_args(q, k_cache, v_cache, cache_seqlens, num_splits, causal, window, softcap,
                      softmax_scale, rescale_threshold, out, lse, block_table, alibi_slopes)
    _check(lib().attn_fwd_kvcache_noalloc(ctypes.byref(a), _stream(stream, q.device)),
           "attn_fwd_kvcache_noalloc")
    return out, lse


ATTN_NOALLOC_SCRATCH_BYTES = 64 << 20


def attn_bwd_workspace_bytes(batch, seqlen_q, heads_q):
    return int(lib().attn_bwd_workspace_bytes(batch, seqlen_q, heads_q))


def _same_dtype(ref, *ts):
    for t in ts:
        if t.dtype != ref.dtype:
            raise TypeError("q, k, v, o, dout and the gradients must share one dtype")
        if t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")


def attn_bwd(q, k, v, o, lse, dout, causal=False, window=(-1, -1), softcap=0.0, softmax_scale=None,
             dq=None, dk=None, dv=None, workspace=None, stream=None, alibi_slopes=None):
    """Gradients of attn_fwd: q, o, dout [B, Sq, Hq, D], k, v [B, Sk, Hkv, D], lse [B, Hq, Sq]
    (from attn_fwd with the same options) -> (dq, dk, dv)."""
    _need_gpu(q, k, v, o, lse, dout)
    b, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    _same_dtype(q, k, v, o, dout, dq, dk, dv)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (b, hq, sq):
        raise TypeError("lse must be a contiguous float32 [batch, heads_q, seqlen_q] tensor")
    need = attn_bwd_workspace_bytes(b, sq, hq)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    a = BwdArgs(_dtype_code(q), b, sq, sk, hq, hkv, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                *[s for t in (q, k, v, o, dout, dq, dk, dv) for s in t.stride()[:3]],
                _opts(causal, window, softcap, softmax_scale, -1.0, alibi_slopes))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().attn_bwd(ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(stream, q.device)), "attn_bwd")
    return dq, dk, dv


def attn_bwd_varlen_workspace_bytes(total_q, heads_q):
    return int(lib().attn_bwd_varlen_workspace_bytes(total_q, heads_q))


def attn_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    causal=False, window=(-1, -1), softcap=0.0, softmax_scale=None, dq=None, dk=None,
                    dv=None, workspace=None, stream=None, alibi_slopes=None):
    """Gradients of attn_fwd_varlen: q, o, dout [Tq, Hq, D], k, v [Tk, Hkv, D], lse [Hq, Tq]."""
    _need_gpu(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k)
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    batch = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    _same_dtype(q, k, v, o, dout, dq, dk, dv)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (hq, tq):
        raise TypeError("lse must be a contiguous float32 [heads_q, total_q] tensor")
    need = attn_bwd_varlen_workspace_bytes(tq, hq)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    a = BwdVarlenArgs(_dtype_code(q), batch, tq, tk, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d,
                      _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                      _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                      *[s for t in (q, k, v, o, dout, dq, dk, dv) for s in t.stride()[:2]],
                      _opts(causal, window, softcap, softmax_scale, -1.0, alibi_slopes))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().attn_bwd_varlen(ctypes.byref(a), _ptr(workspace), ws_bytes, _stream(stream, q.device)),
           "attn_bwd_varlen")
    return dq, dk, dv
