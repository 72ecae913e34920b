"""Accuracy metrics used by the parity gates -- TEST INFRASTRUCTURE.

The gates come from page "v1.7 / flash_attn 2.9.2.post1", section 4
(fp16 rel_Linf <= 2e-2, bf16 rel_Linf <= 1e-2, cosine >= 0.9995).  The page
does not spell the metrics out; the readings used here are:

* rel_Linf = max|O - O_ref| / max|O_ref| over the whole tensor (the ratio of
  the page's printed max_abs and rel_Linf columns in section 4.3 matches
  this reading, while an elementwise ratio would blow up near zero);
* cosine = <O, O_ref> / (|O| |O_ref|) over the flattened tensors, in fp64;
* LSE error = max |LSE - LSE_ref| over rows whose reference is finite; rows
  whose reference is -inf must be -inf exactly.
"""

import numpy as np

__all__ = ["rel_linf", "cosine", "lse_max_abs_err", "compare", "GATES"]

GATES = {
    "fp16": {"rel_linf": 2e-2, "cosine": 0.9995, "lse_abs": 1e-3},
    "bf16": {"rel_linf": 1e-2, "cosine": 0.9995, "lse_abs": 1e-3},
}


def rel_linf(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(out - ref)) if ref.size else 0.0
    if denom == 0.0:
        return float(num)
    return float(num / denom)


def cosine(out, ref):
    a = np.asarray(out, dtype=np.float64).ravel()
    b = np.asarray(ref, dtype=np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0.0 and nb == 0.0:
        return 1.0
    if na == 0.0 or nb == 0.0:
        return 0.0
    return float(np.dot(a, b) / (na * nb))


def lse_max_abs_err(lse, ref):
    """Max abs error on finite reference rows; inf if the -inf pattern differs."""
    lse = np.asarray(lse, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ref_inf = np.isneginf(ref)
    if not np.array_equal(ref_inf, np.isneginf(lse)):
        return float("inf")
    fin = ~ref_inf
    if not fin.any():
        return 0.0
    return float(np.max(np.abs(lse[fin] - ref[fin])))


def compare(out, ref, lse=None, lse_ref=None, dtype="bf16"):
    """All gate metrics plus a pass flag for the given 16-bit dtype."""
    out = np.asarray(out, dtype=np.float64)
    res = {
        "finite": bool(np.all(np.isfinite(out))),
        "rel_linf": rel_linf(out, ref),
        "cosine": cosine(out, ref),
        "max_abs": float(np.max(np.abs(out - np.asarray(ref, dtype=np.float64)))) if out.size else 0.0,
    }
    gate = GATES[dtype]
    ok = res["finite"] and res["rel_linf"] <= gate["rel_linf"] and res["cosine"] >= gate["cosine"]
    if lse is not None:
        res["lse_abs"] = lse_max_abs_err(lse, lse_ref)
        ok = ok and res["lse_abs"] <= gate["lse_abs"]
    res["pass"] = bool(ok)
    return res
