"""Exact tiled attention forward for AMD MI355X (gfx950).

A C-ABI HIP library (``libattn_mi355x.so``, header ``include/attn_mi355x.h``)
with three entry points -- ``attn_fwd`` (causal / sliding window / softcap /
GQA), ``attn_fwd_varlen`` (packed sequences via cu_seqlens) and
``attn_fwd_kvcache`` (split-KV decode plus a log-sum-exp combine) -- and a
thin ctypes binding with the same names.  PyTorch provides device memory and
streams only.
"""

from .binding import (  # noqa: F401
    ATTN_DTYPE_BF16,
    ATTN_DTYPE_F16,
    attn_fwd,
    attn_fwd_kvcache,
    attn_fwd_varlen,
    attn_kvcache_num_splits,
    attn_kvcache_workspace_bytes,
    attn_varlen_workspace_bytes,
    lib,
    status_string,
)
