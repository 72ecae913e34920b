"""Tiled online softmax with RescaleThreshold and max lagging, in fp64 -- TEST INFRASTRUCTURE.

Used only by tests (to pin the method's semantics against the plain
definition in ``attention.py``).  Parity status: pinned -- it must equal
``attention_ref`` to rounding for every threshold and tile size, and its
non-lagging variant must fail in the way the v1.7 page predicts.

The algorithm, in the pages' order (page "FA2 2.9.0 Kernel Changes in v1.2",
sections 1-3, as amended by page "v1.7 / flash_attn 2.9.2.post1", sections
1.1-1.2).  Per query row keep a running max m, a running sum l and an
unnormalised output O (m = -inf, l = 0, O = 0 before the first KV tile).
For each KV tile of ``block_k`` keys, with t the (scaled, capped, masked)
scores of the tile:

1. m_cur = max(m, max over the tile of t).
2. On the first tile (Is_first) nothing is rescaled; m = m_cur.
3. On later tiles, with the -inf guard of the v1.2 page (a -inf max reads
   as 0): scaled_diff = (m - m_cur) * log2(e), in log2 units of the scaled
   score.  If scaled_diff >= -tau the rescale is skipped and m keeps its
   previous value (max lagging, v1.7 Delta 6).  Otherwise
   alpha = exp2(scaled_diff), l *= alpha, O *= alpha and m = m_cur.
4. P = exp2(t * log2(e) - m~ * log2(e)) with m~ = 0 when m = -inf, so with
   lagging P <= exp2(tau); l += row sum of P; O += P V_tile.

Finally O /= l and LSE = m~ + ln(l); a row with l = 0 gives O = 0 and
LSE = -inf.  ``lagging=False`` is the superseded v1.2 rule (on a skip keep
the new max); it is kept only to show that it is wrong at tau = 8.

Per-row statistics (``return_row_stats``).  A tile is *live* for a row when
the row sees at least one key of it.  On a row's first live tile the running
max leaves -inf ("first"); on every later live tile step 3 either skips
(the max lags) or rescales.  So first + skips + rescales = the number of
live tiles of the row, and max_p is the largest P the row ever forms.
Tiles with no visible key change nothing and are not counted.
"""

import numpy as np

from .attention import allowed_mask, kv_head_of, transformed_scores

__all__ = ["tiled_ref", "round_to_16bit"]

LOG2E = 1.0 / np.log(2.0)


def round_to_16bit(x, kind):
    """Round fp64 values to fp16 or bf16 (round to nearest even) and back to fp64."""
    if kind is None:
        return x
    if kind == "fp16":
        return x.astype(np.float16).astype(np.float64)
    if kind == "bf16":
        f = np.ascontiguousarray(x, dtype=np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
        out = rounded.astype(np.uint32).view(np.float32).astype(np.float64)
        return np.where(np.isnan(f), np.nan, out)
    raise ValueError(kind)


def _tiled_one_head(q_h, k_g, v_g, scale, causal, window, softcap, tau, block_k, lagging,
                    order, p_round, stats, row_stats=None):
    seqlen_q, seqlen_k = q_h.shape[0], k_g.shape[0]
    rows = np.arange(seqlen_q)
    m = np.full(seqlen_q, -np.inf)
    l = np.zeros(seqlen_q)
    acc = np.zeros((seqlen_q, v_g.shape[1]))
    starts = list(range(0, seqlen_k, block_k))
    if order == "descending":
        starts = starts[::-1]
    ok_all = allowed_mask(seqlen_q, seqlen_k, rows, causal, window[0], window[1])
    for step, j0 in enumerate(starts):
        j1 = min(j0 + block_k, seqlen_k)
        t = transformed_scores(q_h, k_g[j0:j1], scale, softcap)
        ok = ok_all[:, j0:j1]
        t = np.where(ok, t, -np.inf)
        live = ok.any(axis=1)
        first = live & np.isneginf(m)
        m_cur = np.maximum(m, t.max(axis=1))
        skip = np.zeros(seqlen_q, dtype=bool)
        if step == 0:
            m = m_cur
        else:
            m_cur_guard = np.where(np.isneginf(m_cur), 0.0, m_cur)
            with np.errstate(invalid="ignore"):
                scaled_diff = (m - m_cur_guard) * LOG2E
            skip = scaled_diff >= -tau
            alpha = np.where(skip, 1.0, np.exp2(scaled_diff))
            l = l * alpha
            acc = acc * alpha[:, None]
            if lagging:
                m = np.where(skip, m, m_cur)
            else:
                m = m_cur
            stats["skips"] += int(np.sum(skip & np.isfinite(m_cur)))
            stats["rescales"] += int(np.sum(~skip & np.isfinite(m_cur)))
        m_guard = np.where(np.isneginf(m), 0.0, m)
        p = np.exp2(t * LOG2E - (m_guard * LOG2E)[:, None])
        stats["max_p"] = max(stats["max_p"], float(p.max(initial=0.0)))
        if row_stats is not None:
            later = live & ~first
            row_stats["first"] += first
            row_stats["skips"] += later & skip
            row_stats["rescales"] += later & ~skip
            row_stats["max_p"] = np.maximum(row_stats["max_p"], p.max(axis=1, initial=0.0))
        l = l + p.sum(axis=1)
        acc = acc + round_to_16bit(p, p_round) @ v_g[j0:j1]
    live = l > 0
    out = np.where(live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
    m_guard = np.where(np.isneginf(m), 0.0, m)
    lse = np.where(live, m_guard + np.log(np.where(live, l, 1.0)), -np.inf)
    return out, lse


def tiled_ref(q, k, v, scale=None, causal=False, window=(-1, -1), softcap=0.0, tau=8.0,
              block_k=64, lagging=True, order="ascending", p_round=None, return_stats=False,
              return_row_stats=False):
    """The tiled algorithm above, fp64, for q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D].

    Returns (O [B, Sq, Hq, D], LSE [B, Hq, Sq]) and, with ``return_stats``, a
    dict with the number of skipped and applied rescales and the largest P.
    With ``return_row_stats`` one more dict follows: int arrays "first",
    "skips", "rescales" and float array "max_p", each [B, Hq, Sq] (see the
    module docstring for what is counted).
    ``p_round`` in {None, "fp16", "bf16"} rounds P before the P V product
    (the row sum keeps the unrounded P), to model a 16-bit P operand.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    batch, seqlen_q, heads_q, dim = q.shape
    heads_kv = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(dim)
    out = np.zeros((batch, seqlen_q, heads_q, v.shape[3]))
    lse = np.full((batch, heads_q, seqlen_q), -np.inf)
    stats = {"skips": 0, "rescales": 0, "max_p": 0.0}
    rows = {"first": np.zeros((batch, heads_q, seqlen_q), dtype=np.int64),
            "skips": np.zeros((batch, heads_q, seqlen_q), dtype=np.int64),
            "rescales": np.zeros((batch, heads_q, seqlen_q), dtype=np.int64),
            "max_p": np.zeros((batch, heads_q, seqlen_q))}
    for b in range(batch):
        for h in range(heads_q):
            g = kv_head_of(h, heads_q, heads_kv)
            rs = None
            if return_row_stats:
                rs = {"first": np.zeros(seqlen_q, dtype=np.int64),
                      "skips": np.zeros(seqlen_q, dtype=np.int64),
                      "rescales": np.zeros(seqlen_q, dtype=np.int64),
                      "max_p": np.zeros(seqlen_q)}
            o_bh, lse_bh = _tiled_one_head(q[b, :, h], k[b, :, g], v[b, :, g], scale, causal,
                                           window, softcap, tau, block_k, lagging, order,
                                           p_round, stats, rs)
            out[b, :, h] = o_bh
            lse[b, h] = lse_bh
            if rs is not None:
                for key in rows:
                    rows[key][b, h] = rs[key]
    res = (out, lse)
    if return_stats:
        res = res + (stats,)
    if return_row_stats:
        res = res + (rows,)
    return res
