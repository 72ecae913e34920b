"""Helpers shared by the GPU parity tests (comparison against the CPU oracle)."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def np64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def gate_check(out, ref, lse=None, lse_ref=None, dtype="bf16", what=""):
    """Assert the parity gates: rel_Linf (per dtype), cosine >= 0.9995, LSE abs error <= 1e-3."""
    res = oracle.compare(out, ref, lse, lse_ref, dtype=dtype)
    print(f"[parity] {what}: {res}", flush=True)
    assert res["finite"], f"{what}: non-finite output"
    assert res["pass"], f"{what}: {res}"
    return res


def gpu_required():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_tiled_attention_fa2_amd import binding
    binding.lib()  # fails loudly if the library is missing


def force_variants(request, fwd=0, dec=0, bwd=0):
    """Run this test's library calls on the debug build with the given tile overrides (undone at
    the end of the test).  The release library has no overrides: its kernel choice depends on the
    call's arguments alone."""
    from exact_tiled_attention_fa2_amd import debug
    cm = debug.forced_variants(fwd=fwd, dec=dec, bwd=bwd)
    cm.__enter__()
    request.addfinalizer(lambda: cm.__exit__(None, None, None))


def run_jobs(fn, jobs, workers=None):
    """fn over jobs on a thread pool (at most 16 threads, one BLAS thread each), in order.

    The oracle is NumPy: its matrix products and elementwise passes release
    the GIL, so whole-output references of the full-size workloads are
    computed one (batch, head) at a time in parallel."""
    from threadpoolctl import threadpool_limits
    workers = workers or max(1, min(16, os.cpu_count() or 1))
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, jobs))


def nan_like(t):
    """A tensor shaped like t, filled with NaN: an output position the library never writes fails
    the finiteness gate."""
    return torch.full_like(t, float("nan"), memory_format=torch.contiguous_format)
