"""ctypes access to the debug build, libattn_mi355x_debug.so (tests and sweeps).

The debug build has every entry point of the release library plus those of
``include/attn_mi355x_debug.h``: tile-shape overrides, ``attn_fwd_stats``,
the forward with per-row counters of the rescale-threshold rule, and
``attn_debug_calib_mfma``, a matrix-core rate calibration.  Nothing in
the product path imports this module.

``forced_variants(fwd, dec, bwd)`` routes the binding's entry points to the
debug library and sets the overrides for the duration of a ``with`` block.
"""

import contextlib
import ctypes
import os

import torch

from . import binding
from .build_lib import DEBUG_LIB_PATH

_DEBUG = None


def debug_lib():
    """The loaded debug library (raises if it has not been built)."""
    global _DEBUG
    if _DEBUG is None:
        if not os.path.exists(DEBUG_LIB_PATH):
            raise RuntimeError(f"{DEBUG_LIB_PATH} is missing: build it with "
                               "`python -m exact_tiled_attention_fa2_amd.build_lib`")
        h = binding.configure(ctypes.CDLL(DEBUG_LIB_PATH))
        h.attn_debug_set_variants.argtypes = [ctypes.c_int32] * 3
        h.attn_debug_set_variants.restype = None
        h.attn_debug_last_block_k.argtypes = []
        h.attn_debug_last_block_k.restype = ctypes.c_int32
        h.attn_fwd_stats.argtypes = [ctypes.POINTER(binding.FwdArgs), ctypes.c_void_p, ctypes.c_void_p]
        h.attn_fwd_stats.restype = ctypes.c_int
        h.attn_debug_calib_mfma.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_void_p]
        h.attn_debug_calib_mfma.restype = ctypes.c_int
        _DEBUG = h
    return _DEBUG


@contextlib.contextmanager
def forced_variants(fwd=0, dec=0, bwd=0):
    """Run the binding's entry points on the debug library with the given tile overrides."""
    h = debug_lib()
    h.attn_debug_set_variants(int(fwd), int(dec), int(bwd))
    binding._OVERRIDE.append(h)
    try:
        yield h
    finally:
        binding._OVERRIDE.pop()
        h.attn_debug_set_variants(0, 0, 0)


def last_block_k():
    return int(debug_lib().attn_debug_last_block_k())


def attn_fwd_stats(q, k, v, causal=False, window=(-1, -1), softcap=0.0, softmax_scale=None,
                   rescale_threshold=-1.0, alibi_slopes=None, stream=None):
    """attn_fwd on the debug library plus its per-row counters.

    Returns (o, lse, stats) with stats int32 [B, Hq, Sq, 4]: first-max steps,
    skipped rescales, applied rescales, and the bits of the row's largest fp32
    P (view the last column as float32 for the value).
    """
    binding._need_gpu(q, k, v)
    b, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    out = torch.empty_like(q, memory_format=torch.contiguous_format)
    lse = torch.empty((b, hq, sq), dtype=torch.float32, device=q.device)
    stats = torch.full((b, hq, sq, 4), -1, dtype=torch.int32, device=q.device)
    a = binding.FwdArgs(binding._dtype_code(q), b, sq, sk, hq, hkv, d, binding._ptr(q), binding._ptr(k),
                        binding._ptr(v), binding._ptr(out), binding._ptr(lse),
                        *q.stride()[:3], *k.stride()[:3], *v.stride()[:3], *out.stride()[:3],
                        binding._opts(causal, window, softcap, softmax_scale, rescale_threshold,
                                      alibi_slopes))
    if q.stride(3) != 1 or k.stride(3) != 1 or v.stride(3) != 1:
        raise ValueError("the head dimension must be contiguous")
    binding._check(debug_lib().attn_fwd_stats(ctypes.byref(a), binding._ptr(stats),
                                              binding._stream(stream, q.device)), "attn_fwd_stats")
    return out, lse, stats
