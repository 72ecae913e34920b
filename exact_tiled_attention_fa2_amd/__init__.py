"""Exact tiled attention for AMD MI355X (gfx950).

A C-ABI HIP library (``libattn_mi355x.so``, header ``include/attn_mi355x.h``)
with the forward entry points ``attn_fwd`` (causal / sliding window / softcap /
ALiBi / GQA), ``attn_fwd_varlen`` (packed sequences via cu_seqlens) and
``attn_fwd_kvcache`` (split-KV decode plus a log-sum-exp combine, contiguous
or paged cache; ``attn_fwd_kvcache_noalloc`` is the same without a workspace,
for callers that cannot allocate), the backward entry points ``attn_bwd`` and
``attn_bwd_varlen`` (dQ, dK, dV from the saved LSE), and a thin ctypes
binding with the same names.  PyTorch provides device memory and streams
only.
"""

from .binding import (  # noqa: F401
    ATTN_DTYPE_BF16,
    ATTN_DTYPE_F16,
    attn_bwd,
    attn_bwd_varlen,
    attn_bwd_varlen_workspace_bytes,
    attn_bwd_workspace_bytes,
    attn_fwd,
    attn_fwd_kvcache,
    attn_fwd_kvcache_noalloc,
    attn_fwd_varlen,
    attn_kvcache_num_splits,
    attn_kvcache_workspace_bytes,
    attn_varlen_workspace_bytes,
    lib,
    status_string,
)
