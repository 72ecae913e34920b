"""Helpers shared by the GPU parity tests (comparison against the CPU oracle)."""

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


def sample_rows(n_rows, count, seed):
    """Sorted unique query rows: the first, the last, and random ones in between."""
    rng = np.random.default_rng(seed)
    rows = set([0, n_rows - 1])
    rows.update(rng.integers(0, n_rows, size=count).tolist())
    return np.array(sorted(rows), dtype=np.int64)
