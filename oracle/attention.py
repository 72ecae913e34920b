"""Plain definition of exact attention forward, in fp64 -- TEST INFRASTRUCTURE.

Only tests, the smoke check and the benchmark's cpu_baseline leg use this
module; the GPU library never does.  Parity status: pinned (see
``tests/test_oracle_pins.py``: closed forms, invariants, brute force and the
special cases printed on the pages).

What is computed.  The method of the v1.7 fork release (page "v1.7 /
flash_attn 2.9.2.post1", section 1.2) tiles the softmax with a running max
and, when it skips a rescale, keeps the previous max so that O, row_sum and P
share one base; the page states that output and LSE are then exact.  So the
oracle is the plain definition the tiled method reaches, written out with
the whole score row materialised:

    s_ij = scale * <Q_i, K_j>                       (scaled dot product)
    t_ij = cap * tanh(s_ij / cap)  if cap > 0       (softcap; else t = s)
    LSE_i = ln sum_{j allowed} exp(t_ij)            (natural log, fp64)
    O_i   = sum_{j allowed} exp(t_ij - LSE_i) * V_j
    a row with no allowed key: O_i = 0, LSE_i = -inf

Readings where the pages are silent:

* causal and window masks are aligned to the bottom-right corner,
  off = Sk - Sq; key j is allowed for query i iff
  (not causal or j <= i + off) and (left < 0 or j >= i + off - left) and
  (right < 0 or j <= i + off + right).  A bound of -1 means unbounded and a
  bound of 0 is a real zero-width bound (aichaai page, release notes of
  fa4-v4.0.0.beta30); window (0,0) therefore leaves only the diagonal, which
  gives O == V as the v1.7 page's section 4.6 probe reports.
* softcap is applied to the scaled score, before the mask.
* GQA: query head h reads KV head h // (Hq / Hkv) (contiguous groups).
* LSE is in natural-log units with layout [B, Hq, Sq] (v1.7 section 4.6
  gives the shape; its printed range fits natural log).
* ALiBi (named among the public API features, v1.7 section 2, and in its
  API-path table, section 4; no formula is printed): the plainest reading,
  -slope_h * |i + off - j| added to t_ij after the softcap and before the
  mask, with a slope per query head (optionally per batch entry).
"""

import numpy as np

__all__ = [
    "kv_head_of",
    "allowed_mask",
    "transformed_scores",
    "alibi_bias",
    "attention_ref",
    "attention_varlen_ref",
    "attention_kvcache_ref",
    "sequence_slopes",
]


def kv_head_of(h, heads_q, heads_kv):
    """KV head read by query head ``h`` under GQA/MQA (contiguous groups)."""
    if heads_q % heads_kv != 0:
        raise ValueError("heads_q must be a multiple of heads_kv")
    return h // (heads_q // heads_kv)


def allowed_mask(seqlen_q, seqlen_k, rows, causal=False, window_left=-1, window_right=-1):
    """Boolean [len(rows), seqlen_k]: True where key j may be attended by query row i.

    Bottom-right aligned: off = seqlen_k - seqlen_q.  Window bounds < 0 are
    unbounded; 0 is a real bound.
    """
    off = seqlen_k - seqlen_q
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(seqlen_k, dtype=np.int64)[None, :]
    ok = np.ones((i.shape[0], seqlen_k), dtype=bool)
    if causal:
        ok &= j <= i + off
    if window_left >= 0:
        ok &= j >= i + off - window_left
    if window_right >= 0:
        ok &= j <= i + off + window_right
    return ok


def transformed_scores(q_rows, k_mat, scale, softcap=0.0):
    """t = scale * Q K^T, then cap * tanh(t / cap) when softcap > 0 (fp64)."""
    s = scale * (q_rows @ k_mat.T)
    if softcap > 0.0:
        s = softcap * np.tanh(s / softcap)
    return s


def alibi_bias(seqlen_q, seqlen_k, rows, slope):
    """-slope * |i + off - j| for query rows ``rows`` and every key j (off = Sk - Sq)."""
    off = seqlen_k - seqlen_q
    i = np.asarray(rows, dtype=np.float64)[:, None]
    j = np.arange(seqlen_k, dtype=np.float64)[None, :]
    return -float(slope) * np.abs(i + off - j)


def _one_head(q_h, k_g, v_g, rows, scale, causal, window_left, window_right, softcap,
              chunk, want_probs, alibi_slope=None):
    """Exact attention of query rows ``rows`` of one head against one KV head.

    q_h [Sq, D], k_g/v_g [Sk, D] in fp64.  Returns O [R, D], LSE [R] and,
    when asked, P [R, Sk].  Rows are processed in independent chunks only to
    bound memory; each row's result depends on that row alone.
    """
    seqlen_q, seqlen_k = q_h.shape[0], k_g.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], v_g.shape[1]), dtype=np.float64)
    lse = np.full((rows.shape[0],), -np.inf, dtype=np.float64)
    probs = np.zeros((rows.shape[0], seqlen_k), dtype=np.float64) if want_probs else None
    if seqlen_k == 0:
        return out, lse, probs
    for c0 in range(0, rows.shape[0], chunk):
        r = rows[c0:c0 + chunk]
        t = transformed_scores(q_h[r], k_g, scale, softcap)
        if alibi_slope is not None:
            t = t + alibi_bias(seqlen_q, seqlen_k, r, alibi_slope)
        ok = allowed_mask(seqlen_q, seqlen_k, r, causal, window_left, window_right)
        t = np.where(ok, t, -np.inf)
        has_key = ok.any(axis=1)
        m = np.where(has_key, t.max(axis=1, initial=-np.inf), 0.0)
        e = np.exp(t - m[:, None])                       # exp(-inf) = 0 on masked keys
        total = e.sum(axis=1)
        row_lse = np.where(has_key, m + np.log(np.where(has_key, total, 1.0)), -np.inf)
        p = np.where(has_key[:, None], np.exp(t - np.where(has_key, row_lse, 0.0)[:, None]), 0.0)
        out[c0:c0 + chunk] = p @ v_g
        lse[c0:c0 + chunk] = row_lse
        if want_probs:
            probs[c0:c0 + chunk] = p
    return out, lse, probs


def _slope(alibi_slopes, b, h):
    if alibi_slopes is None:
        return None
    a = np.asarray(alibi_slopes, dtype=np.float64)
    return a[h] if a.ndim == 1 else a[b, h]


def attention_ref(q, k, v, scale=None, causal=False, window=(-1, -1), softcap=0.0,
                  rows=None, return_probs=False, chunk=512, alibi_slopes=None):
    """Exact attention forward, plain definition, fp64.

    q [B, Sq, Hq, D]; k, v [B, Sk, Hkv, D] (any real dtype, upcast to fp64).
    ``scale`` defaults to 1/sqrt(D).  ``window`` = (left, right), -1 for
    unbounded.  ``rows`` optionally restricts the computation to those query
    rows (outputs then hold only those rows, in that order).
    ``alibi_slopes`` [Hq] or [B, Hq] adds the ALiBi distance bias.

    Returns (O [B, R, Hq, D], LSE [B, Hq, R]) and, with ``return_probs``, the
    probability matrix P [B, Hq, R, Sk].  R = Sq unless ``rows`` is given.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    batch, seqlen_q, heads_q, dim = q.shape
    seqlen_k, heads_kv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(dim)
    rows = np.arange(seqlen_q) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((batch, rows.shape[0], heads_q, v.shape[3]), dtype=np.float64)
    lse = np.full((batch, heads_q, rows.shape[0]), -np.inf, dtype=np.float64)
    probs = np.zeros((batch, heads_q, rows.shape[0], seqlen_k)) if return_probs else None
    for b in range(batch):
        for h in range(heads_q):
            g = kv_head_of(h, heads_q, heads_kv)
            o_bh, lse_bh, p_bh = _one_head(q[b, :, h, :], k[b, :, g, :], v[b, :, g, :], rows,
                                           scale, causal, window[0], window[1], softcap,
                                           chunk, return_probs, _slope(alibi_slopes, b, h))
            out[b, :, h, :] = o_bh
            lse[b, h, :] = lse_bh
            if return_probs:
                probs[b, h] = p_bh
    if return_probs:
        return out, lse, probs
    return out, lse


def sequence_slopes(alibi_slopes, b):
    """ALiBi slopes for the one-sequence call of batch entry (or packed sequence) b.

    ``alibi_slopes`` is None, [Hq] (one slope per query head, shared by every
    sequence) or [B, Hq] (row b belongs to sequence b).  Returns None, the
    [Hq] array unchanged, or row b as a [1, Hq] array for a batch-1 call.
    """
    if alibi_slopes is None:
        return None
    a = np.asarray(alibi_slopes, dtype=np.float64)
    return a if a.ndim == 1 else a[b:b + 1]


def _batch_entry(kw, b):
    """Keyword arguments for the one-sequence call of batch entry b (per-batch ALiBi slopes)."""
    if kw.get("alibi_slopes") is None:
        return kw
    kw = dict(kw)
    kw["alibi_slopes"] = sequence_slopes(kw["alibi_slopes"], b)
    return kw


def attention_varlen_ref(q, k, v, cu_seqlens_q, cu_seqlens_k, **kw):
    """Packed variable-length attention: each sequence attends only to itself.

    q [Tq, Hq, D], k/v [Tk, Hkv, D]; cu_seqlens_* are prefix sums [B+1]
    starting at 0.  Sequence b occupies rows cu[b]..cu[b+1]-1.  Returns
    (O [Tq, Hq, D], LSE [Hq, Tq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    out = np.zeros((q.shape[0], q.shape[1], v.shape[2]), dtype=np.float64)
    lse = np.full((q.shape[1], q.shape[0]), -np.inf, dtype=np.float64)
    for b in range(cu_q.shape[0] - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if q1 == q0:
            continue
        o_b, lse_b = attention_ref(q[None, q0:q1], k[None, k0:k1], v[None, k0:k1],
                                   **_batch_entry(kw, b))
        out[q0:q1] = o_b[0]
        lse[:, q0:q1] = lse_b[0]
    return out, lse


def gather_pages(pool, table_row, n):
    """Rows 0..n-1 of one sequence of a paged cache, in key order.

    pool [num_pages, page_size, Hkv, D]; table_row[i] is the page holding keys
    i*page_size .. (i+1)*page_size - 1 (the paged KV cache of the Python API,
    "flash-attention" project survey page, csrc/flash_attn entry; the layout
    is the reading taken here).  Only the pages covering the first n keys are
    read.
    """
    page = pool.shape[1]
    npages = -(-n // page)
    rows = [pool[int(table_row[i])] for i in range(npages)]
    if not rows:
        return np.zeros((0,) + pool.shape[2:], dtype=pool.dtype)
    return np.concatenate(rows, axis=0)[:n]


def attention_kvcache_ref(q, k_cache, v_cache, cache_seqlens=None, block_table=None, **kw):
    """Attention of q [B, Sq, Hq, D] against the first cache_seqlens[b] rows of a cache.

    k_cache/v_cache [B, Sk_max, Hkv, D], or with block_table [B, pages_per_seq]
    a page pool [num_pages, page_size, Hkv, D] (see gather_pages).  Entries at
    or beyond the valid length are not read at all (they may hold NaN).
    Returns (O [B, Sq, Hq, D], LSE [B, Hq, Sq]).
    """
    q = np.asarray(q, dtype=np.float64)
    batch = q.shape[0]
    if cache_seqlens is None:
        cap = k_cache.shape[1] if block_table is None else len(block_table[0]) * k_cache.shape[1]
        cache_seqlens = [cap] * batch
    out = np.zeros(q.shape[:3] + (v_cache.shape[3],), dtype=np.float64)
    lse = np.full((batch, q.shape[2], q.shape[1]), -np.inf, dtype=np.float64)
    for b in range(batch):
        n = int(cache_seqlens[b])
        if block_table is None:
            kb = np.asarray(k_cache[b:b + 1, :n], dtype=np.float64)
            vb = np.asarray(v_cache[b:b + 1, :n], dtype=np.float64)
        else:
            kb = np.asarray(gather_pages(k_cache, block_table[b], n), dtype=np.float64)[None]
            vb = np.asarray(gather_pages(v_cache, block_table[b], n), dtype=np.float64)[None]
        o_b, lse_b = attention_ref(q[b:b + 1], kb, vb, **_batch_entry(kw, b))
        out[b] = o_b[0]
        lse[b] = lse_b[0]
    return out, lse
