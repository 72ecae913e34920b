"""Plant plausible mistakes in the oracle (on the CPU) and check that some pin catches each.

This shows the pins are strong enough: a dropped scale, an off-by-one mask,
top-left instead of bottom-right alignment, a wrong GQA head map, a
transposed operand, softcap on the unscaled score, log2 instead of natural
log, a missing max shift, a window bound read as unbounded, the superseded
keep-new-max skip rule, or a backward without the softmax row term, the
softcap derivative, the scale or the GQA sum must each make at least one pin
fail.  So must a slip in the gate code every GPU verdict passes through (an
"or" for an "and", a dropped cosine or LSE gate, a loosened bf16
gate, a wrong cosine normaliser) and a wrong per-sequence ALiBi slope row.
"""

import contextlib

import numpy as np
import pytest

import oracle_pins
from oracle import attention as oatt
from oracle import backward as obwd
from oracle import tiled as otiled

_orig_mask = oatt.allowed_mask
_orig_scores = oatt.transformed_scores
_orig_head = oatt.kv_head_of
_orig_one_head = oatt._one_head
_orig_tiled_one = otiled._tiled_one_head


def _mask_causal_strict(sq, sk, rows, causal=False, wl=-1, wr=-1):
    ok = _orig_mask(sq, sk, rows, False, wl, wr)
    if causal:
        i = np.asarray(rows)[:, None]
        j = np.arange(sk)[None, :]
        ok &= j < i + (sk - sq)
    return ok


def _mask_top_left(sq, sk, rows, causal=False, wl=-1, wr=-1):
    return _orig_mask(sk, sk, rows, causal, wl, wr)


def _mask_window_zero_unbounded(sq, sk, rows, causal=False, wl=-1, wr=-1):
    return _orig_mask(sq, sk, rows, causal, -1 if wl == 0 else wl, -1 if wr == 0 else wr)


def _mask_left_off_by_one(sq, sk, rows, causal=False, wl=-1, wr=-1):
    return _orig_mask(sq, sk, rows, causal, wl + 1 if wl >= 0 else wl, wr)


def _scores_no_scale(qr, km, scale, softcap=0.0):
    return _orig_scores(qr, km, 1.0, softcap)


def _scores_transposed(qr, km, scale, softcap=0.0):
    s = scale * (qr @ km.T)
    s = s[:, ::-1]                       # keys read in the wrong order
    if softcap > 0:
        s = softcap * np.tanh(s / softcap)
    return s


def _scores_cap_before_scale(qr, km, scale, softcap=0.0):
    s = qr @ km.T
    if softcap > 0:
        s = softcap * np.tanh(s / softcap)
    return scale * s


def _head_modulo(h, hq, hkv):
    return h % hkv


def _one_head_log2(*a, **kw):
    o, l, p = _orig_one_head(*a, **kw)
    return o, l / np.log(2.0), p


def _one_head_no_max_shift(q_h, k_g, v_g, rows, scale, causal, wl, wr, softcap, chunk, want):
    out = np.zeros((len(rows), v_g.shape[1]))
    lse = np.full(len(rows), -np.inf)
    probs = np.zeros((len(rows), k_g.shape[0])) if want else None
    t = oatt.transformed_scores(q_h[rows], k_g, scale, softcap)
    ok = oatt.allowed_mask(q_h.shape[0], k_g.shape[0], rows, causal, wl, wr)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.where(ok, np.exp(t), 0.0)
        z = e.sum(axis=1)
        p = e / z[:, None]
        out[:] = p @ v_g
        lse[:] = np.log(z)
    if want:
        probs[:] = p
    return out, lse, probs


def _tiled_no_lagging(*a, **kw):
    a = list(a)
    a[9] = False                          # lagging flag position in _tiled_one_head
    return _orig_tiled_one(*a, **kw)


def _tiled_natural_exp(q_h, k_g, v_g, scale, causal, window, softcap, tau, block_k, lagging,
                       order, p_round, stats, row_stats=None):
    saved = otiled.LOG2E
    otiled.LOG2E = 1.0                    # exp2 of the raw score: wrong base
    try:
        return _orig_tiled_one(q_h, k_g, v_g, scale, causal, window, softcap, tau, block_k,
                               lagging, order, p_round, stats, row_stats)
    finally:
        otiled.LOG2E = saved


def _gather_row_shift(pool, table_row, n):
    page = pool.shape[1]
    flat = np.concatenate([pool[int(table_row[i])] for i in range(len(table_row))], axis=0)
    return flat[1:n + 1] if n + 1 <= len(flat) else flat[:n]      # off by one row


def _gather_page_order(pool, table_row, n):
    page = pool.shape[1]
    npages = -(-n // page)
    rows = [pool[i] for i in range(npages)]                      # table ignored: pool order
    return np.concatenate(rows, axis=0)[:n]


def _alibi_sign(seqlen_q, seqlen_k, rows, slope):
    return -_orig_alibi(seqlen_q, seqlen_k, rows, slope)         # bias added with the wrong sign


def _alibi_no_offset(seqlen_q, seqlen_k, rows, slope):
    return _orig_alibi(seqlen_k, seqlen_k, rows, slope)          # distance |i - j|, top-left


def _alibi_scaled(seqlen_q, seqlen_k, rows, slope):
    return _orig_alibi(seqlen_q, seqlen_k, rows, slope) * 0.5    # bias in pre-scale units


_orig_alibi = oatt.alibi_bias


def _bwd_no_rowsum(p, dp):
    return p * dp                                                # softmax Jacobian without the row term


def _bwd_no_softcap_factor(dt, u, scale, softcap):
    return scale * dt                                            # tanh derivative dropped


def _bwd_softcap_factor_linear(dt, u, scale, softcap):
    if softcap > 0.0:
        dt = dt * (1.0 - np.abs(np.tanh(u / softcap)))           # 1 - |tanh| instead of 1 - tanh^2
    return scale * dt


def _bwd_no_scale(dt, u, scale, softcap):
    if softcap > 0.0:
        th = np.tanh(u / softcap)
        dt = dt * (1.0 - th * th)
    return dt                                                    # d<Q,K> missing the scale


def _bwd_gqa_overwrite(dk, dv, dk_h, dv_h):
    dk[...] = dk_h                                               # last query head wins
    dv[...] = dv_h


from oracle import metrics as omet

_orig_compare = omet.compare
_orig_cosine = omet.cosine


def _compare_variant(use_or=False, cosine_gate=True, finite_gate=True, lse_gate=True):
    def compare(out, ref, lse=None, lse_ref=None, dtype="bf16"):
        out = np.asarray(out, dtype=np.float64)
        res = {"finite": bool(np.all(np.isfinite(out))), "rel_linf": omet.rel_linf(out, ref),
               "cosine": omet.cosine(out, ref)}
        gate = omet.GATES[dtype]
        r_ok = res["rel_linf"] <= gate["rel_linf"]
        c_ok = res["cosine"] >= gate["cosine"] if cosine_gate else True
        f_ok = res["finite"] if finite_gate else True
        ok = (r_ok or c_ok) if use_or else (r_ok and c_ok)
        ok = ok and f_ok
        if lse is not None:
            res["lse_abs"] = omet.lse_max_abs_err(lse, lse_ref)
            if lse_gate:
                ok = ok and res["lse_abs"] <= gate["lse_abs"]
        res["pass"] = bool(ok)
        return res
    return compare


def _cosine_sq_norm(out, ref):
    a = np.asarray(out, dtype=np.float64).ravel()
    b = np.asarray(ref, dtype=np.float64).ravel()
    na = np.linalg.norm(a)
    return float(np.dot(a, b) / (na * na)) if na else 0.0     # |a|^2 instead of |a||b|


_LOOSE_GATES = {"fp16": {"rel_linf": 2e-2, "cosine": 0.9995, "lse_abs": 1e-3},
                "bf16": {"rel_linf": 2e-2, "cosine": 0.9995, "lse_abs": 1e-3}}


def _slopes_first_sequence(alibi_slopes, b):
    if alibi_slopes is None:
        return None
    a = np.asarray(alibi_slopes, dtype=np.float64)
    return a if a.ndim == 1 else a[0:1]                          # row 0 for every sequence


MUTATIONS = {
    "compare_or_for_and": (omet, "compare", _compare_variant(use_or=True)),
    "compare_no_cosine_gate": (omet, "compare", _compare_variant(cosine_gate=False)),
    "compare_lse_ignored": (omet, "compare", _compare_variant(lse_gate=False)),
    "gates_bf16_loosened": (omet, "GATES", _LOOSE_GATES),
    "cosine_sq_norm": (omet, "cosine", _cosine_sq_norm),
    "alibi_first_sequence_slopes": (oatt, "sequence_slopes", _slopes_first_sequence),
    "causal_strict_lt": (oatt, "allowed_mask", _mask_causal_strict),
    "top_left_alignment": (oatt, "allowed_mask", _mask_top_left),
    "window_zero_as_unbounded": (oatt, "allowed_mask", _mask_window_zero_unbounded),
    "window_left_off_by_one": (oatt, "allowed_mask", _mask_left_off_by_one),
    "dropped_scale": (oatt, "transformed_scores", _scores_no_scale),
    "keys_reversed": (oatt, "transformed_scores", _scores_transposed),
    "softcap_before_scale": (oatt, "transformed_scores", _scores_cap_before_scale),
    "gqa_modulo_map": (oatt, "kv_head_of", _head_modulo),
    "lse_log2_units": (oatt, "_one_head", _one_head_log2),
    "no_max_shift": (oatt, "_one_head", _one_head_no_max_shift),
    "tiled_keep_new_max": (otiled, "_tiled_one_head", _tiled_no_lagging),
    "tiled_wrong_exp_base": (otiled, "_tiled_one_head", _tiled_natural_exp),
    "paged_row_off_by_one": (oatt, "gather_pages", _gather_row_shift),
    "paged_table_ignored": (oatt, "gather_pages", _gather_page_order),
    "alibi_sign": (oatt, "alibi_bias", _alibi_sign),
    "alibi_no_offset": (oatt, "alibi_bias", _alibi_no_offset),
    "alibi_scaled": (oatt, "alibi_bias", _alibi_scaled),
    "bwd_no_rowsum": (obwd, "softmax_backward", _bwd_no_rowsum),
    "bwd_no_softcap_factor": (obwd, "score_backward", _bwd_no_softcap_factor),
    "bwd_softcap_factor_linear": (obwd, "score_backward", _bwd_softcap_factor_linear),
    "bwd_no_scale": (obwd, "score_backward", _bwd_no_scale),
    "bwd_gqa_overwrite": (obwd, "_add_kv_grad", _bwd_gqa_overwrite),
}


@contextlib.contextmanager
def _patched(mod, name, fn):
    old = getattr(mod, name)
    setattr(mod, name, fn)
    try:
        yield
    finally:
        setattr(mod, name, old)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    mod, attr, fn = MUTATIONS[name]
    caught = []
    with _patched(mod, attr, fn):
        for pin in oracle_pins.ALL_PINS:
            try:
                with np.errstate(all="ignore"):
                    pin()
            except Exception:            # AssertionError or a crash: the pin caught it
                caught.append(pin.__name__)
    assert caught, f"mutation {name} passed every pin"
