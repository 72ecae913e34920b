"""Plain definition of the attention backward, in fp64 -- TEST INFRASTRUCTURE.

Only tests and the smoke check use this module; the GPU library never does.
Parity status: pinned (``tests/test_oracle_pins.py``: fp64 torch autograd of
an independently written forward, central finite differences of the pinned
forward, and the invariants of the softmax Jacobian).

What is computed.  The pages list a backward pass (dQ, dK, dV) among the
library's kernels and check its gradients against an fp32 reference (page
"v1.7 / flash_attn 2.9.2.post1", section 4.4); they print no formula, so the
oracle is the gradient of the forward definition (``attention.py``) for the
loss L = sum(dO * O), per batch entry and query head:

    u_ij = scale * <Q_i, K_j>
    t_ij = cap * tanh(u_ij / cap)  if cap > 0, else u_ij
    t_ij += bias_ij (ALiBi) ; t_ij = -inf where key j is not allowed
    P_i  = softmax_j(t_i)          (zero row when no key is allowed)
    O_i  = sum_j P_ij V_j

    dV_j  = sum_i P_ij dO_i
    dP_ij = <dO_i, V_j>
    dT_ij = P_ij (dP_ij - sum_k P_ik dP_ik)          (softmax Jacobian)
    dU_ij = dT_ij (1 - tanh(u_ij / cap)^2)  if cap > 0, else dT_ij
    dQ_i  = scale * sum_j dU_ij K_j
    dK_j  = scale * sum_i dU_ij Q_i

The ALiBi bias does not depend on Q or K and adds no term.  Under GQA a KV
head's dK and dV sum the contributions of all query heads that read it.
Masks, alignment, window and softcap follow the forward's readings.
"""

import numpy as np

from . import attention as _attention
from .attention import allowed_mask, alibi_bias, kv_head_of, _slope

__all__ = [
    "softmax_backward",
    "score_backward",
    "attention_bwd_ref",
    "attention_bwd_varlen_ref",
]


def softmax_backward(p, dp):
    """dT = P * (dP - rowsum(P * dP)): the softmax Jacobian applied to dP, row by row."""
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def score_backward(dt, u, scale, softcap):
    """dL/d<Q_i, K_j> from dL/dt: the softcap chain rule, then the scale."""
    if softcap > 0.0:
        th = np.tanh(u / softcap)
        dt = dt * (1.0 - th * th)
    return scale * dt


def _add_kv_grad(dk, dv, dk_h, dv_h):
    """GQA: the KV head's gradients sum over the query heads that read it."""
    dk += dk_h
    dv += dv_h


def _one_head_bwd(q_h, k_g, v_g, do_h, scale, causal, window_left, window_right, softcap,
                  alibi_slope):
    """Gradients of one query head against one KV head: (dQ [Sq, D], dK [Sk, D], dV [Sk, Dv])."""
    seqlen_q, seqlen_k = q_h.shape[0], k_g.shape[0]
    dq = np.zeros_like(q_h)
    dk = np.zeros_like(k_g)
    dv = np.zeros_like(v_g)
    if seqlen_q == 0 or seqlen_k == 0:
        return dq, dk, dv
    rows = np.arange(seqlen_q)
    u = scale * (q_h @ k_g.T)
    t = softcap * np.tanh(u / softcap) if softcap > 0.0 else u.copy()
    if alibi_slope is not None:
        t = t + alibi_bias(seqlen_q, seqlen_k, rows, alibi_slope)
    ok = allowed_mask(seqlen_q, seqlen_k, rows, causal, window_left, window_right)
    t = np.where(ok, t, -np.inf)
    has_key = ok.any(axis=1)
    m = np.where(has_key, t.max(axis=1, initial=-np.inf), 0.0)
    e = np.exp(t - m[:, None])
    total = np.where(has_key, e.sum(axis=1), 1.0)
    p = np.where(has_key[:, None], e / total[:, None], 0.0)
    dv = p.T @ do_h
    dp = do_h @ v_g.T
    dt = softmax_backward(p, dp)
    du = score_backward(dt, u, scale, softcap)
    dq = du @ k_g
    dk = du.T @ q_h
    return dq, dk, dv


def attention_bwd_ref(q, k, v, do, scale=None, causal=False, window=(-1, -1), softcap=0.0,
                      alibi_slopes=None):
    """Backward of ``attention_ref`` for the loss sum(dO * O), plain definition, fp64.

    q, do [B, Sq, Hq, D]; k, v [B, Sk, Hkv, D].  Same options as the forward.
    Returns (dQ [B, Sq, Hq, D], dK [B, Sk, Hkv, D], dV [B, Sk, Hkv, D]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    batch, seqlen_q, heads_q, dim = q.shape
    heads_kv = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(dim)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(batch):
        for h in range(heads_q):
            g = kv_head_of(h, heads_q, heads_kv)
            dq_h, dk_h, dv_h = _one_head_bwd(q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h],
                                             scale, causal, window[0], window[1], softcap,
                                             _slope(alibi_slopes, b, h))
            dq[b, :, h] = dq_h
            _add_kv_grad(dk[b, :, g], dv[b, :, g], dk_h, dv_h)
    return dq, dk, dv


def attention_bwd_varlen_ref(q, k, v, do, cu_seqlens_q, cu_seqlens_k, **kw):
    """Backward of ``attention_varlen_ref``: each packed sequence on its own.

    q, do [Tq, Hq, D]; k, v [Tk, Hkv, D]; cu_seqlens_* [B+1].  Returns
    (dQ [Tq, Hq, D], dK [Tk, Hkv, D], dV [Tk, Hkv, D]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    slopes = kw.pop("alibi_slopes", None)
    for b in range(cu_q.shape[0] - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        sl = _attention.sequence_slopes(slopes, b)
        dq_b, dk_b, dv_b = attention_bwd_ref(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1],
                                             do[None, q0:q1], alibi_slopes=sl, **kw)
        dq[q0:q1] = dq_b[0]
        dk[k0:k1] = dk_b[0]
        dv[k0:k1] = dv_b[0]
    return dq, dk, dv
