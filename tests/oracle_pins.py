"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function raises AssertionError (or any exception) when the
oracle disagrees with a closed form, an invariant, a brute-force evaluation,
a library routine or a number printed on the pages.  ``test_oracle_pins.py``
runs them; ``test_oracle_mutations.py`` plants plausible mistakes in the
oracle and checks that some pin catches each one.

Page citations: [v1.7] = release page "v1.7 / flash_attn 2.9.2.post1";
[v1.2] = release page "FA2 2.9.0 Kernel Changes in v1.2"; [aichaai] =
Dao-AILab/flash-attention project page (release notes).
"""

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import attention as oatt
from oracle import metrics as ometrics
from oracle import tiled as otiled

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _visible_count(i, sq, sk, causal, left, right):
    """Closed-form number of visible keys of row i (bottom-right aligned band)."""
    off = sk - sq
    hi = sk - 1
    lo = 0
    if causal:
        hi = min(hi, i + off)
    if right >= 0:
        hi = min(hi, i + off + right)
    if left >= 0:
        lo = max(lo, i + off - left)
    return max(0, hi - lo + 1), lo, hi


# ---------------------------------------------------------------- closed forms

def pin_uniform_scores():
    """Q = 0 makes every score 0 (and tanh(0) = 0): O_i = mean of the visible V_j, LSE_i = ln n_i."""
    rng = _rng(1)
    cases = [
        dict(sq=24, sk=24, causal=False, window=(-1, -1), softcap=0.0),
        dict(sq=24, sk=24, causal=True, window=(-1, -1), softcap=0.0),
        dict(sq=16, sk=40, causal=True, window=(-1, -1), softcap=30.0),
        dict(sq=40, sk=16, causal=True, window=(-1, -1), softcap=0.0),
        dict(sq=30, sk=30, causal=False, window=(5, 3), softcap=0.0),
        dict(sq=20, sk=33, causal=True, window=(7, -1), softcap=5.0),
        dict(sq=12, sk=12, causal=False, window=(0, 0), softcap=0.0),
    ]
    for c in cases:
        q = np.zeros((1, c["sq"], 2, 8))
        k = rng.standard_normal((1, c["sk"], 1, 8))
        v = rng.standard_normal((1, c["sk"], 1, 8))
        out, lse = oracle.attention_ref(q, k, v, scale=0.3, causal=c["causal"], window=c["window"],
                                        softcap=c["softcap"])
        for i in range(c["sq"]):
            n, lo, hi = _visible_count(i, c["sq"], c["sk"], c["causal"], *c["window"])
            for h in range(2):
                if n == 0:
                    assert np.all(out[0, i, h] == 0.0) and lse[0, h, i] == -np.inf, (c, i)
                else:
                    mean = v[0, lo:hi + 1, 0].sum(axis=0) / n
                    assert np.allclose(out[0, i, h], mean, rtol=0, atol=1e-13), (c, i)
                    assert abs(lse[0, h, i] - math.log(n)) < 1e-13, (c, i)


def pin_one_hot_scores():
    """Orthogonal keys with a margin of 800 nats: O_i = V_pi(i), LSE_i = t_i,pi(i)."""
    rng = _rng(2)
    sk, d = 16, 32
    alpha, beta, scale = 4.0, 200.0, 1.0         # margin 800 nats: exp overflows without a max shift
    k = np.zeros((1, sk, 1, d))
    for j in range(sk):
        k[0, j, 0, j] = alpha                        # K_j = alpha * e_j
    v = rng.standard_normal((1, sk, 1, d))
    perm = rng.permutation(sk)
    q = np.zeros((1, sk, 1, d))
    for i in range(sk):
        q[0, i, 0, perm[i]] = beta                   # <Q_i, K_j> = alpha*beta*[j == perm[i]]
    out, lse = oracle.attention_ref(q, k, v, scale=scale)
    for i in range(sk):
        assert np.allclose(out[0, i, 0], v[0, perm[i], 0], rtol=0, atol=1e-12)
        assert abs(lse[0, 0, i] - alpha * beta * scale) < 1e-12
    # causal: row i sees keys 0..i, and the hot key is i itself
    q2 = np.zeros((1, sk, 1, d))
    for i in range(sk):
        q2[0, i, 0, i] = beta
    out2, lse2 = oracle.attention_ref(q2, k, v, scale=scale, causal=True)
    for i in range(sk):
        assert np.allclose(out2[0, i, 0], v[0, i, 0], rtol=0, atol=1e-12)
        assert abs(lse2[0, 0, i] - alpha * beta * scale) < 1e-12


def pin_softcap_single_key():
    """Window (0,0) leaves one key, so LSE_i = cap * tanh(scale * <Q_i, K_i> / cap) exactly."""
    rng = _rng(3)
    s, d, cap, scale = 10, 16, 2.5, 0.7
    q = rng.standard_normal((1, s, 1, d)) * 2.0
    k = rng.standard_normal((1, s, 1, d)) * 2.0
    v = rng.standard_normal((1, s, 1, d))
    _, lse = oracle.attention_ref(q, k, v, scale=scale, window=(0, 0), softcap=cap)
    for i in range(s):
        dot = math.fsum(float(q[0, i, 0, x]) * float(k[0, i, 0, x]) for x in range(d))
        assert abs(lse[0, 0, i] - cap * math.tanh(scale * dot / cap)) < 1e-12
    # |t| < cap always, and cap -> infinity reduces to no softcap
    out_a, lse_a = oracle.attention_ref(q * 10, k, v, softcap=cap)
    _, _, p = oracle.attention_ref(q * 10, k, v, softcap=cap, return_probs=True)
    assert np.all(np.isfinite(lse_a))
    assert np.all(lse_a <= cap + math.log(s) + 1e-12)
    out_b, lse_b = oracle.attention_ref(q, k, v, softcap=1e9)
    out_c, lse_c = oracle.attention_ref(q, k, v)
    assert np.allclose(out_b, out_c, atol=1e-9) and np.allclose(lse_b, lse_c, atol=1e-9)


# ---------------------------------------------------------------- invariants

def pin_rows_sum_to_one():
    """P >= 0, each row with visible keys sums to 1, and P = 0 exactly off the visible band."""
    rng = _rng(4)
    for (sq, sk, causal, window) in [(20, 20, True, (-1, -1)), (13, 29, True, (4, -1)),
                                     (25, 25, False, (3, 6)), (30, 11, True, (-1, -1))]:
        q = rng.standard_normal((1, sq, 1, 8))
        k = rng.standard_normal((1, sk, 1, 8))
        v = rng.standard_normal((1, sk, 1, 8))
        _, lse, p = oracle.attention_ref(q, k, v, causal=causal, window=window, return_probs=True)
        assert np.all(p >= 0)
        for i in range(sq):
            n, lo, hi = _visible_count(i, sq, sk, causal, *window)
            row = p[0, 0, i]
            if n == 0:
                assert np.all(row == 0) and lse[0, 0, i] == -np.inf
                continue
            assert abs(row.sum() - 1.0) < 1e-13
            assert np.count_nonzero(row) == n
            assert np.all(row[:lo] == 0) and np.all(row[hi + 1:] == 0)


def pin_permutation_invariance():
    """Without a mask, permuting the (K_j, V_j) pairs jointly leaves O and LSE unchanged."""
    rng = _rng(5)
    q = rng.standard_normal((2, 9, 4, 16))
    k = rng.standard_normal((2, 23, 2, 16))
    v = rng.standard_normal((2, 23, 2, 16))
    perm = rng.permutation(23)
    o1, l1 = oracle.attention_ref(q, k, v, softcap=3.0)
    o2, l2 = oracle.attention_ref(q, k[:, perm], v[:, perm], softcap=3.0)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


def pin_bruteforce_tiny():
    """Python-float evaluation (math.fsum, no max shift) of LSE and O for tiny shapes."""
    rng = _rng(6)
    for (sq, sk, causal, window, cap) in [(5, 7, True, (-1, -1), 0.0), (6, 6, False, (1, 2), 0.0),
                                          (4, 9, False, (-1, -1), 1.5), (7, 3, True, (2, -1), 0.0)]:
        d, scale = 4, 0.9
        q = rng.standard_normal((1, sq, 1, d))
        k = rng.standard_normal((1, sk, 1, d))
        v = rng.standard_normal((1, sk, 1, d))
        out, lse = oracle.attention_ref(q, k, v, scale=scale, causal=causal, window=window,
                                        softcap=cap)
        off = sk - sq
        for i in range(sq):
            ws = []
            for j in range(sk):
                visible = True
                if causal and j > i + off:
                    visible = False
                if window[0] >= 0 and j < i + off - window[0]:
                    visible = False
                if window[1] >= 0 and j > i + off + window[1]:
                    visible = False
                if not visible:
                    continue
                s = scale * math.fsum(float(q[0, i, 0, x]) * float(k[0, j, 0, x]) for x in range(d))
                if cap > 0:
                    s = cap * math.tanh(s / cap)
                ws.append((math.exp(s), j))
            if not ws:
                assert lse[0, 0, i] == -np.inf and np.all(out[0, i, 0] == 0)
                continue
            z = math.fsum(w for w, _ in ws)
            assert abs(lse[0, 0, i] - math.log(z)) < 1e-13
            for x in range(d):
                ref = math.fsum(w * float(v[0, j, 0, x]) for w, j in ws) / z
                assert abs(out[0, i, 0, x] - ref) < 1e-13


def pin_lse_reconstructs_output():
    """exp(LSE) equals the sum of exp(t) by brute force; O equals the LSE-weighted V sum."""
    rng = _rng(7)
    q = rng.standard_normal((1, 11, 1, 8))
    k = rng.standard_normal((1, 11, 1, 8))
    v = rng.standard_normal((1, 11, 1, 8))
    out, lse, p = oracle.attention_ref(q, k, v, causal=True, return_probs=True)
    # P rows are the softmax of the visible scores: P_ij / P_i0 = exp(t_ij - t_i0)
    for i in range(11):
        t = (q[0, i, 0] @ k[0, :i + 1, 0].T) / math.sqrt(8)
        assert np.allclose(p[0, 0, i, :i + 1] / p[0, 0, i, 0], np.exp(t - t[0]), rtol=1e-12)
        assert abs(lse[0, 0, i] - (t[0] - math.log(p[0, 0, i, 0]))) < 1e-12
    assert np.allclose(out[0, :, 0], p[0, 0] @ v[0, :, 0], atol=1e-13)


# ---------------------------------------------------------------- page special cases

def pin_page_window_00_is_v():
    """[v1.7] section 4.6: window (0,0) gives output == V (max abs diff 0)."""
    probe = _golden("page_v17_probes.json")
    rng = _rng(8)
    q = rng.standard_normal((2, 64, 4, 16))
    k = rng.standard_normal((2, 64, 2, 16))
    v = rng.standard_normal((2, 64, 2, 16))
    out, _ = oracle.attention_ref(q, k, v, window=(0, 0))
    vv = np.repeat(v, 2, axis=2)
    assert np.max(np.abs(out - vv)) == probe["window_0_0_max_abs_diff_vs_v"]


def pin_page_single_row_and_causal_row0():
    """[v1.7] section 4.6 S=1 probe and causal row 0: one visible key, O = V_0 and LSE = t_00."""
    rng = _rng(9)
    q = rng.standard_normal((1, 1, 1, 16))
    k = rng.standard_normal((1, 1, 1, 16))
    v = rng.standard_normal((1, 1, 1, 16))
    out, lse = oracle.attention_ref(q, k, v)
    assert np.array_equal(out[0, 0, 0], v[0, 0, 0])
    assert abs(lse[0, 0, 0] - float(q[0, 0, 0] @ k[0, 0, 0]) / 4.0) < 1e-13
    q = rng.standard_normal((1, 32, 1, 16))
    k = rng.standard_normal((1, 32, 1, 16))
    v = rng.standard_normal((1, 32, 1, 16))
    out, _ = oracle.attention_ref(q, k, v, causal=True)
    assert np.array_equal(out[0, 0, 0], v[0, 0, 0])


def pin_page_lse_units():
    """[v1.7] section 4.6 LSE probe: shape [B, H, S]; its top end fits natural-log units."""
    probe = _golden("page_v17_probes.json")["lse_probe"]
    b, h, s, d = probe["batch"], probe["heads"], probe["seqlen"], probe["head_dim"]
    rng = _rng(10)
    q = np.zeros((b, s, h, d))
    k = rng.standard_normal((b, s, h, d))
    v = rng.standard_normal((b, s, h, d))
    _, lse = oracle.attention_ref(q, k, v, causal=True)
    assert list(lse.shape) == probe["shape"]
    lo, hi = probe["range"]
    assert abs(lse.max() - hi) < 0.01          # ln(512) = 6.2383; log2 would give 9.0
    assert abs(lse.min() - lo) < 0.03


def pin_decode_is_last_prefill_row():
    """A one-row query against a cache equals the last row of causal prefill on the same K/V."""
    rng = _rng(11)
    q = rng.standard_normal((2, 17, 4, 16))
    k = rng.standard_normal((2, 17, 2, 16))
    v = rng.standard_normal((2, 17, 2, 16))
    out, lse = oracle.attention_ref(q, k, v, causal=True)
    kc = np.concatenate([k, np.full((2, 5, 2, 16), np.nan)], axis=1)   # NaN past the valid length
    vc = np.concatenate([v, np.full((2, 5, 2, 16), np.nan)], axis=1)
    o1, l1 = oracle.attention_kvcache_ref(q[:, -1:], kc, vc, cache_seqlens=[17, 17], causal=True)
    assert np.allclose(o1[:, 0], out[:, -1], atol=1e-13)
    assert np.allclose(l1[:, :, 0], lse[:, :, -1], atol=1e-13)


def pin_paged_cache_is_contiguous():
    """A paged cache (pages scattered over a shuffled pool, the rest NaN) gives exactly the
    result of the contiguous cache it pages, for lengths that end inside a page."""
    rng = _rng(12)
    b, sk, hkv, hq, d, page = 3, 20, 2, 4, 8, 4
    q = rng.standard_normal((b, 2, hq, d))
    k = rng.standard_normal((b, sk, hkv, d))
    v = rng.standard_normal((b, sk, hkv, d))
    lens = [13, 20, 1]
    per = sk // page
    pool_k = np.full((b * per + 3, page, hkv, d), np.nan)
    pool_v = np.full((b * per + 3, page, hkv, d), np.nan)
    slots = rng.permutation(b * per + 3)
    table = np.zeros((b, per), dtype=np.int64)
    for bi in range(b):
        for i in range(per):
            s_ = int(slots[bi * per + i])
            table[bi, i] = s_
            rows = slice(i * page, (i + 1) * page)
            kk, vv = k[bi, rows].copy(), v[bi, rows].copy()
            past = np.arange(i * page, (i + 1) * page) >= lens[bi]
            kk[past] = np.nan                       # rows past the valid length are never read
            vv[past] = np.nan
            pool_k[s_], pool_v[s_] = kk, vv
    for causal in (False, True):
        o_c, l_c = oracle.attention_kvcache_ref(q, k, v, cache_seqlens=lens, causal=causal)
        o_p, l_p = oracle.attention_kvcache_ref(q, pool_k, pool_v, cache_seqlens=lens,
                                                block_table=table, causal=causal)
        assert np.array_equal(o_c, o_p) and np.array_equal(l_c, l_p)
    # the gather itself, row by row
    for bi in range(b):
        g = oracle.gather_pages(pool_k, table[bi], lens[bi])
        assert np.array_equal(g, k[bi, :lens[bi]])


def pin_alibi_closed_forms():
    """ALiBi with Q = 0: every raw score is 0, so t_ij = -slope |i + off - j| and the weights
    are geometric.  LSE_i = ln sum_d exp(-slope d) over the visible distances, O_i the matching
    weighted mean of V (weights written out independently of the oracle)."""
    rng = _rng(13)
    slope = 0.37
    for (sq, sk, causal) in [(9, 9, True), (9, 9, False), (3, 11, True), (1, 7, False)]:
        q = np.zeros((1, sq, 2, 8))
        k = rng.standard_normal((1, sk, 1, 8))
        v = rng.standard_normal((1, sk, 1, 8))
        out, lse = oracle.attention_ref(q, k, v, causal=causal, alibi_slopes=[slope, 2 * slope])
        off = sk - sq
        for h, sl in ((0, slope), (1, 2 * slope)):
            for i in range(sq):
                js = [j for j in range(sk) if (not causal or j <= i + off)]
                w = [math.exp(-sl * abs(i + off - j)) for j in js]
                tot = math.fsum(w)
                assert abs(lse[0, h, i] - math.log(tot)) < 1e-12
                o_ref = sum(wj * v[0, j, 0] for wj, j in zip(w, js)) / tot
                assert np.allclose(out[0, i, h], o_ref, atol=1e-12)
    # per-batch slopes [B, Hq] equal the [Hq] form when the rows agree
    q = rng.standard_normal((2, 5, 2, 8))
    k = rng.standard_normal((2, 5, 2, 8))
    v = rng.standard_normal((2, 5, 2, 8))
    o1, l1 = oracle.attention_ref(q, k, v, causal=True, alibi_slopes=[0.5, 0.25])
    o2, l2 = oracle.attention_ref(q, k, v, causal=True, alibi_slopes=[[0.5, 0.25], [0.5, 0.25]])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = oracle.attention_ref(q, k, v, causal=True, alibi_slopes=[[0.5, 0.25], [0.0, 0.0]])
    o4, l4 = oracle.attention_ref(q, k, v, causal=True)
    assert np.array_equal(o3[1], o4[1]) and np.array_equal(l3[1], l4[1])


def pin_alibi_after_softcap():
    """One query, two keys, softcap 2: t_j = cap tanh(scale s_j / cap) - slope d_j, bias after
    the cap (a cap applied to the biased score gives another LSE)."""
    d = 4
    q = np.zeros((1, 1, 1, d)); q[0, 0, 0, 0] = 3.0
    k = np.zeros((1, 2, 1, d)); k[0, 0, 0, 0] = 1.5; k[0, 1, 0, 0] = -0.5
    v = np.zeros((1, 2, 1, d)); v[0, 0, 0, 1] = 1.0; v[0, 1, 0, 2] = 1.0
    scale, cap, slope = 0.5, 2.0, 0.8
    _, lse = oracle.attention_ref(q, k, v, scale=scale, softcap=cap, alibi_slopes=[slope])
    t0 = cap * math.tanh(scale * 4.5 / cap) - slope * 1.0     # key 0: distance off - 0 = 1
    t1 = cap * math.tanh(scale * -1.5 / cap) - slope * 0.0    # key 1: distance 0
    assert abs(lse[0, 0, 0] - math.log(math.exp(t0) + math.exp(t1))) < 1e-13


# ---------------------------------------------------------------- backward

def _torch_attention(q, k, v, scale, causal, window, softcap, slopes):
    """An independent fp64 torch forward (autograd-ready): masks by masked_fill, GQA by
    repeat_interleave, softcap by torch.tanh, ALiBi from a distance matrix."""
    b, sq, hq, d = q.shape
    sk, hkv = k.shape[1], k.shape[2]
    g = hq // hkv
    qt = q.permute(0, 2, 1, 3)
    kt = k.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    vt = v.repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    s = torch.matmul(qt, kt.transpose(-1, -2)) * scale
    if softcap > 0:
        s = softcap * torch.tanh(s / softcap)
    i = torch.arange(sq, dtype=torch.float64)[:, None] + (sk - sq)
    j = torch.arange(sk, dtype=torch.float64)[None, :]
    if slopes is not None:
        sl = torch.as_tensor(slopes, dtype=torch.float64)
        sl = sl[None, :, None, None] if sl.ndim == 1 else sl[:, :, None, None]
        s = s - sl * (i - j).abs()
    keep = torch.ones(sq, sk, dtype=torch.bool)
    if causal:
        keep &= j <= i
    if window[0] >= 0:
        keep &= j >= i - window[0]
    if window[1] >= 0:
        keep &= j <= i + window[1]
    s = s.masked_fill(~keep, float("-inf"))
    return torch.matmul(torch.softmax(s, dim=-1), vt).permute(0, 2, 1, 3)


def pin_bwd_autograd():
    """dQ, dK, dV = fp64 torch autograd of an independently written forward (causal, window,
    softcap, ALiBi, GQA, Sq != Sk; every row keeps at least one key)."""
    rng = _rng(21)
    cases = [
        (2, 9, 9, 4, 2, 8, dict(causal=True)),
        (1, 7, 12, 2, 2, 16, dict(causal=True, softcap=1.5)),
        (2, 11, 11, 6, 3, 8, dict(causal=False, window=(3, 2))),
        (1, 10, 10, 4, 1, 8, dict(causal=True, window=(4, 0), softcap=2.0, slopes=[0.3, 0.1, 0.7, 0.05])),
        (2, 8, 8, 2, 2, 8, dict(causal=False, slopes=[[0.2, 0.5], [0.9, 0.0]])),
    ]
    for (b, sq, sk, hq, hkv, d, kw) in cases:
        q = rng.standard_normal((b, sq, hq, d))
        k = rng.standard_normal((b, sk, hkv, d))
        v = rng.standard_normal((b, sk, hkv, d))
        do = rng.standard_normal((b, sq, hq, d))
        scale = 0.6
        causal, window = kw.get("causal", False), kw.get("window", (-1, -1))
        softcap, slopes = kw.get("softcap", 0.0), kw.get("slopes")
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = _torch_attention(tq, tk, tv, scale, causal, window, softcap, slopes)
        (o * torch.from_numpy(do)).sum().backward()
        dq, dk, dv = oracle.attention_bwd_ref(q, k, v, do, scale=scale, causal=causal, window=window,
                                              softcap=softcap, alibi_slopes=slopes)
        for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.allclose(mine, ref.numpy(), atol=1e-11, rtol=1e-11)


def pin_bwd_finite_differences():
    """Central differences of sum(dO * O) through the (pinned) forward oracle, every input
    coordinate of a tiny causal, windowed, softcapped, ALiBi, GQA problem."""
    rng = _rng(22)
    b, sq, sk, hq, hkv, d = 1, 4, 6, 2, 1, 3
    q = rng.standard_normal((b, sq, hq, d))
    k = rng.standard_normal((b, sk, hkv, d))
    v = rng.standard_normal((b, sk, hkv, d))
    do = rng.standard_normal((b, sq, hq, d))
    kw = dict(scale=0.8, causal=True, window=(3, -1), softcap=1.7, alibi_slopes=[0.25, 0.6])

    def loss(q_, k_, v_):
        o, _ = oracle.attention_ref(q_, k_, v_, **kw)
        return float((o * do).sum())

    dq, dk, dv = oracle.attention_bwd_ref(q, k, v, do, **kw)
    h = 1e-5
    for x, grad, slot in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        for idx in np.ndindex(x.shape):
            args = [q, k, v]
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args[slot] = xp
            fp = loss(*args)
            args[slot] = xm
            fm = loss(*args)
            assert abs((fp - fm) / (2 * h) - grad[idx]) < 1e-7, (slot, idx)


def pin_bwd_invariants():
    """Softmax Jacobian facts: sum_j dV_j = sum of dO over rows with a key; without softcap
    sum_j dK_j = 0 and dQ does not change when every K row moves by the same vector; rows
    with no visible key get dQ = 0 and add nothing to dK, dV."""
    rng = _rng(23)
    b, sq, sk, hq, hkv, d = 2, 12, 9, 4, 2, 8
    q = rng.standard_normal((b, sq, hq, d))
    k = rng.standard_normal((b, sk, hkv, d))
    v = rng.standard_normal((b, sk, hkv, d))
    do = rng.standard_normal((b, sq, hq, d))
    kw = dict(causal=True, alibi_slopes=[0.1, 0.2, 0.3, 0.4])
    dq, dk, dv = oracle.attention_bwd_ref(q, k, v, do, **kw)
    g = hq // hkv
    live = sq - sk   # causal with Sq > Sk: rows 0 .. Sq-Sk-1 see no key
    for bb in range(b):
        for kvh in range(hkv):
            heads = range(kvh * g, (kvh + 1) * g)
            want = sum(do[bb, live:, h].sum(axis=0) for h in heads)
            assert np.allclose(dv[bb, :, kvh].sum(axis=0), want, atol=1e-12)
            assert np.allclose(dk[bb, :, kvh].sum(axis=0), 0.0, atol=1e-12)
    assert np.all(dq[:, :live] == 0.0)
    shift = rng.standard_normal(d)
    dq2, _, _ = oracle.attention_bwd_ref(q, k + shift, v, do, **kw)
    assert np.allclose(dq2, dq, atol=1e-12)
    # the empty rows' dO does not reach dK or dV
    do3 = do.copy()
    do3[:, :live] = rng.standard_normal(do3[:, :live].shape)
    _, dk3, dv3 = oracle.attention_bwd_ref(q, k, v, do3, **kw)
    assert np.array_equal(dk3, dk) and np.array_equal(dv3, dv)


def pin_bwd_varlen_is_per_sequence():
    """Packed-sequence backward = the dense backward of each sequence on its own."""
    rng = _rng(24)
    lens = [5, 1, 0, 8]
    cu = np.concatenate([[0], np.cumsum(lens)])
    hq, hkv, d = 4, 2, 8
    q = rng.standard_normal((cu[-1], hq, d))
    k = rng.standard_normal((cu[-1], hkv, d))
    v = rng.standard_normal((cu[-1], hkv, d))
    do = rng.standard_normal((cu[-1], hq, d))
    dq, dk, dv = oracle.attention_bwd_varlen_ref(q, k, v, do, cu, cu, causal=True)
    for s in range(len(lens)):
        a, z = cu[s], cu[s + 1]
        if z == a:
            continue
        rq, rk, rv = oracle.attention_bwd_ref(q[None, a:z], k[None, a:z], v[None, a:z], do[None, a:z],
                                              causal=True)
        assert np.array_equal(dq[a:z], rq[0]) and np.array_equal(dk[a:z], rk[0])
        assert np.array_equal(dv[a:z], rv[0])


# ---------------------------------------------------------------- library routines

def _sdpa_ref(q, k, v, scale, mask_bool):
    """torch scaled_dot_product_attention in fp64 on the CPU ([B, S, H, D] in, [B, S, H, D] out)."""
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    g = q.shape[2] // k.shape[2]
    kt = torch.from_numpy(np.repeat(k, g, axis=2)).permute(0, 2, 1, 3).contiguous()
    vt = torch.from_numpy(np.repeat(v, g, axis=2)).permute(0, 2, 1, 3).contiguous()
    m = None if mask_bool is None else torch.from_numpy(mask_bool)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def pin_torch_sdpa():
    """The pages' own accuracy reference is PyTorch SDPA; cross-check dense, causal, window and GQA."""
    rng = _rng(12)
    b, s, hq, hkv, d = 2, 37, 6, 2, 16
    q = rng.standard_normal((b, s, hq, d))
    k = rng.standard_normal((b, s, hkv, d))
    v = rng.standard_normal((b, s, hkv, d))
    scale = 0.37
    o, _ = oracle.attention_ref(q, k, v, scale=scale)
    assert np.allclose(o, _sdpa_ref(q, k, v, scale, None), atol=1e-12)
    tri = np.tril(np.ones((s, s), dtype=bool))
    o, _ = oracle.attention_ref(q, k, v, scale=scale, causal=True)
    assert np.allclose(o, _sdpa_ref(q, k, v, scale, tri), atol=1e-12)
    ii, jj = np.meshgrid(np.arange(s), np.arange(s), indexing="ij")
    band = (jj >= ii - 4) & (jj <= ii + 2)
    o, _ = oracle.attention_ref(q, k, v, scale=scale, window=(4, 2))
    assert np.allclose(o, _sdpa_ref(q, k, v, scale, band), atol=1e-12)


def pin_alibi_sdpa():
    """ALiBi = torch SDPA (fp64) with the distance bias passed as an additive float mask, and -inf
    where causal masking hides a key; random inputs, Sq != Sk both ways, GQA."""
    rng = _rng(15)
    for (sq, sk, causal) in [(13, 13, True), (7, 19, True), (19, 7, False), (11, 11, False)]:
        b, hq, hkv, d = 2, 4, 2, 16
        q = rng.standard_normal((b, sq, hq, d))
        k = rng.standard_normal((b, sk, hkv, d))
        v = rng.standard_normal((b, sk, hkv, d))
        slopes = rng.uniform(0.05, 1.0, size=(b, hq))
        scale = 0.3
        out, _ = oracle.attention_ref(q, k, v, scale=scale, causal=causal, alibi_slopes=slopes)
        i = np.arange(sq)[:, None] + (sk - sq)
        j = np.arange(sk)[None, :]
        dist = np.abs(i - j).astype(np.float64)
        for bb in range(b):
            mask = -slopes[bb][:, None, None] * dist[None]          # [Hq, Sq, Sk]
            if causal:
                mask = np.where(j <= i, mask, -np.inf)
            ref = _sdpa_ref(q[bb:bb + 1], k[bb:bb + 1], v[bb:bb + 1], scale, mask[None])
            assert np.allclose(out[bb:bb + 1], ref, atol=1e-12)


def pin_varlen_block_diagonal():
    """Packed sequences = one long sequence under a block-diagonal causal mask (torch SDPA)."""
    rng = _rng(13)
    lens = [5, 1, 12, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    t = int(cu[-1])
    q = rng.standard_normal((t, 4, 8))
    k = rng.standard_normal((t, 2, 8))
    v = rng.standard_normal((t, 2, 8))
    o, lse = oracle.attention_varlen_ref(q, k, v, cu, cu, causal=True)
    mask = np.zeros((t, t), dtype=bool)
    for a, z in zip(cu[:-1], cu[1:]):
        mask[a:z, a:z] = np.tril(np.ones((z - a, z - a), dtype=bool))
    ref = _sdpa_ref(q[None], k[None], v[None], 1.0 / math.sqrt(8), mask)[0]
    assert np.allclose(o, ref, atol=1e-12)
    assert lse.shape == (4, t)


def pin_gqa_is_repeated_mha():
    """GQA equals MHA with each KV head repeated for its group of consecutive query heads."""
    rng = _rng(14)
    q = rng.standard_normal((1, 19, 8, 16))
    k = rng.standard_normal((1, 19, 2, 16))
    v = rng.standard_normal((1, 19, 2, 16))
    o1, l1 = oracle.attention_ref(q, k, v, causal=True)
    o2, l2 = oracle.attention_ref(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- the tiled method

def _ramp_inputs(seed, s=256, d=32, heads=2):
    rng = _rng(seed)
    q = rng.standard_normal((1, s, heads, d))
    k = rng.standard_normal((1, s, heads, d))
    ramp = 1.0 + 3.0 * (np.arange(s) // 32) / (s // 32 - 1)
    k = k * ramp[None, :, None, None]
    v = rng.standard_normal((1, s, heads, d))
    return q, k, v


def pin_tiled_equals_definition():
    """[v1.7] section 1.2: with max lagging any threshold gives the exact output and LSE."""
    q, k, v = _ramp_inputs(15)
    ref_o, ref_l = oracle.attention_ref(q, k, v, causal=True)
    seen_skip = seen_rescale = False
    for tau in (0.0, 8.0):
        for bk in (16, 64, 128):
            for order in ("ascending", "descending"):
                o, l, st = oracle.tiled_ref(q, k, v, causal=True, tau=tau, block_k=bk, order=order,
                                            return_stats=True)
                assert np.max(np.abs(o - ref_o)) < 1e-12 and np.max(np.abs(l - ref_l)) < 1e-12
                if tau == 8.0 and order == "ascending":
                    seen_skip |= st["skips"] > 0
                    seen_rescale |= st["rescales"] > 0
    assert seen_skip and seen_rescale
    for kw in (dict(window=(40, 0)), dict(softcap=3.0), dict(window=(17, 9), causal=False)):
        o, l = oracle.tiled_ref(q, k, v, tau=8.0, block_k=32, **kw)
        ro, rl = oracle.attention_ref(q, k, v, **kw)
        assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(rl - l)) < 1e-12


def _two_block_case(d_log2):
    """Two KV blocks, one key each; the second block's score is higher by d_log2 in log2 units."""
    t1 = 0.3
    t2 = t1 + d_log2 * math.log(2.0)
    q = np.zeros((1, 1, 1, 2))
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 2, 1, 2))
    k[0, 0, 0, 0] = t1
    k[0, 1, 0, 0] = t2
    v = np.zeros((1, 2, 1, 2))
    v[0, 0, 0, 0] = 1.0                                  # block 1 writes into component 0
    v[0, 1, 0, 1] = 1.0                                  # block 2 writes into component 1
    return q, k, v


def pin_page_threshold_numbers():
    """[v1.7] section 1.2 and [v1.2] section 1: the numbers printed about the threshold.

    A max rise of exactly 8 (log2 units) is skipped at tau = 8.  Keeping the
    new max (the superseded rule) then overweights the stale block by
    2^8 = 256; lagging keeps the exact weights and lets P reach exactly 256.
    At the old 0.01 threshold the stale factor is 2^0.01 (scale >= 0.993, error < 0.7%).
    """
    g = _golden("page_v17_threshold.json")
    for d_log2, tau, key in ((8.0, g["tau_16bit"], "overweight_without_lagging_at_tau8"),
                             (0.01, -g["old_threshold"], None)):
        q, k, v = _two_block_case(d_log2)
        exact_ratio = 2.0 ** (-d_log2)                   # w1 / w2 of the exact softmax
        o_lag, _, st = oracle.tiled_ref(q, k, v, scale=1.0, tau=tau, block_k=1,
                                        return_stats=True)
        assert st["skips"] == 1 and st["rescales"] == 0
        assert abs(o_lag[0, 0, 0, 0] / o_lag[0, 0, 0, 1] - exact_ratio) < 1e-12
        o_bad, _ = oracle.tiled_ref(q, k, v, scale=1.0, tau=tau, block_k=1, lagging=False)
        overweight = (o_bad[0, 0, 0, 0] / o_bad[0, 0, 0, 1]) / exact_ratio
        if key is not None:
            assert abs(overweight - g[key]) < 1e-9
            assert abs(st["max_p"] - g["p_bound_with_lagging_at_tau8"]) < 1e-9
            assert st["max_p"] < g["fp16_max"] < g["bf16_max"]
        else:
            assert 1.0 / overweight >= g["old_threshold_min_scale"]
            assert overweight - 1.0 < g["old_threshold_max_rel_error"]


def pin_nonlagging_is_wrong_at_tau8():
    """The superseded keep-new-max rule at tau = 8 is far off on a rising-max input."""
    q, k, v = _ramp_inputs(16)
    ref_o, ref_l = oracle.attention_ref(q, k, v, causal=True)
    o, l = oracle.tiled_ref(q, k, v, causal=True, tau=8.0, block_k=32, lagging=False)
    assert oracle.rel_linf(o, ref_o) > 0.05
    assert np.max(np.abs(l - ref_l)) > 0.5


def pin_p_bound():
    """[v1.7] section 1.2: with lagging at tau = 8, P never exceeds exp2(8) = 256."""
    q, k, v = _ramp_inputs(17, s=512)
    _, _, st = oracle.tiled_ref(q * 3.0, k, v, causal=True, tau=8.0, block_k=32, return_stats=True)
    assert st["max_p"] <= 256.0 + 1e-9 and st["skips"] > 0


def pin_bf16_rounding_helper():
    """round_to_16bit('bf16') is round-to-nearest-even, as torch's own conversion."""
    x = np.random.default_rng(18).standard_normal(4096) * 37.0
    x = np.concatenate([x, [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 256.0, 65504.0]])
    ours = otiled.round_to_16bit(x, "bf16")
    ref = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def pin_metrics():
    """rel_Linf is max|diff| / max|ref| (the page's max_abs / rel_Linf columns agree with this)."""
    ref = np.array([0.5, -0.25, 0.1])
    out = ref + np.array([1e-3, -2e-3, 0.0])
    assert abs(oracle.rel_linf(out, ref) - 2e-3 / 0.5) < 1e-15
    assert abs(oracle.cosine(ref, ref) - 1.0) < 1e-15
    assert oracle.lse_max_abs_err(np.array([-np.inf, 1.0]), np.array([-np.inf, 1.5])) == 0.5
    assert oracle.lse_max_abs_err(np.array([0.0, 1.0]), np.array([-np.inf, 1.0])) == float("inf")


def pin_gates_are_the_pages():
    """[v1.7] section 4: fp16 rel_Linf <= 2e-2, bf16 rel_Linf <= 1e-2, cosine >= 0.9995 (read
    from the golden file of the page's numbers); the LSE gate, 1e-3 absolute, is the stated
    target beside them (the page prints no LSE gate)."""
    g = _golden("page_v17_probes.json")["gates"]
    gates = ometrics.GATES
    assert set(gates) == {"fp16", "bf16"}
    assert gates["fp16"]["rel_linf"] == g["fp16_rel_linf"]
    assert gates["bf16"]["rel_linf"] == g["bf16_rel_linf"]
    for dt in ("fp16", "bf16"):
        assert gates[dt]["cosine"] == g["cosine"]
        assert gates[dt]["lse_abs"] == 1e-3


def pin_cosine_hand_values():
    """Cosine of hand-picked pairs: [1,0].[1,1] = 1/sqrt(2), [3,4].[4,3] = 24/25, opposite
    vectors -1, orthogonal 0; independent of either vector's length."""
    sq2 = 1.0 / math.sqrt(2.0)
    assert abs(ometrics.cosine(np.array([1.0, 0.0]), np.array([1.0, 1.0])) - sq2) < 1e-15
    assert abs(ometrics.cosine(np.array([3.0, 4.0]), np.array([4.0, 3.0])) - 0.96) < 1e-15
    assert abs(ometrics.cosine(np.array([1.0, 2.0, 3.0]), np.array([-1.0, -2.0, -3.0])) + 1.0) < 1e-15
    assert ometrics.cosine(np.array([0.0, 2.0]), np.array([5.0, 0.0])) == 0.0
    a = np.array([[0.3, -1.2], [2.0, 0.7]])
    b = np.array([[1.1, 0.4], [-0.2, 0.9]])
    c0 = ometrics.cosine(a, b)
    assert abs(ometrics.cosine(7.5 * a, b) - c0) < 1e-15 and abs(ometrics.cosine(a, 0.01 * b) - c0) < 1e-15
    dot = 0.3 * 1.1 - 1.2 * 0.4 - 2.0 * 0.2 + 0.7 * 0.9
    na = math.sqrt(0.09 + 1.44 + 4.0 + 0.49)
    nb = math.sqrt(1.21 + 0.16 + 0.04 + 0.81)
    assert abs(c0 - dot / (na * nb)) < 1e-15


def pin_compare_each_gate():
    """compare() passes a case that meets every gate, and fails each hand-built case that
    breaks exactly one of them: non-finite output, rel_Linf (per dtype), cosine, LSE error,
    and the -inf pattern of LSE."""
    ref = np.full(4000, 0.5)
    lref = np.array([0.25, -np.inf, 3.0])
    ok = ometrics.compare(ref.copy(), ref, lref.copy(), lref, dtype="bf16")
    assert ok["pass"] and ok["finite"] and ok["rel_linf"] == 0.0 and ok["lse_abs"] == 0.0
    # a rel_Linf exactly at the gate passes (the gates are inclusive)
    edge = np.array([1.0, 0.0]), np.array([1.0, 0.01])
    assert ometrics.compare(edge[1], edge[0], dtype="bf16")["pass"]
    # non-finite output only
    bad = ref.copy(); bad[17] = np.nan
    assert not ometrics.compare(bad, ref, dtype="fp16")["pass"]
    bad = ref.copy(); bad[3] = np.inf
    r = ometrics.compare(bad, ref, dtype="fp16")
    assert not r["finite"] and not r["pass"]
    # rel_Linf 1.5e-2 with cosine ~ 1: fails the bf16 gate, passes the fp16 gate
    out = ref.copy(); out[0] += 0.0075
    rb, rf = ometrics.compare(out, ref, dtype="bf16"), ometrics.compare(out, ref, dtype="fp16")
    assert abs(rb["rel_linf"] - 0.015) < 1e-12 and rb["cosine"] > 0.99999
    assert not rb["pass"] and rf["pass"]
    # cosine 1/sqrt(1 + 1000 * 0.009^2) = 0.962 with rel_Linf 9e-3: fails on cosine alone
    ref2 = np.zeros(1001); ref2[0] = 1.0
    out2 = np.full(1001, 0.009); out2[0] = 1.0
    r = ometrics.compare(out2, ref2, dtype="bf16")
    assert r["rel_linf"] <= 1e-2 and abs(r["cosine"] - 1.0 / math.sqrt(1.081)) < 1e-12
    assert not r["pass"]
    # LSE off by 2e-3 on one finite row
    l2 = lref.copy(); l2[2] += 2e-3
    r = ometrics.compare(ref.copy(), ref, l2, lref, dtype="fp16")
    assert abs(r["lse_abs"] - 2e-3) < 1e-12 and not r["pass"]
    # -inf pattern: a finite LSE where the reference is -inf, and the reverse
    l3 = lref.copy(); l3[1] = -50.0
    assert not ometrics.compare(ref.copy(), ref, l3, lref, dtype="fp16")["pass"]
    l4 = lref.copy(); l4[0] = -np.inf
    assert not ometrics.compare(ref.copy(), ref, l4, lref, dtype="fp16")["pass"]
    # without an LSE only the output gates apply
    assert ometrics.compare(ref.copy(), ref, dtype="fp16")["pass"]


def pin_alibi_per_sequence_slopes():
    """[B, Hq] ALiBi slopes: packed sequence (or cache entry) b uses row b of the table, in the
    forward (varlen, kv-cache) and in the varlen backward -- each checked against batch-1
    calls of the dense functions written out with that row as [Hq] slopes."""
    rng = _rng(41)
    hq, hkv, d = 4, 2, 8
    table = np.array([[0.5, 0.25, 0.125, 0.0625], [2.0, 0.0, 1.0, 3.0], [0.3, 0.9, 0.05, 1.7]])
    lens = [6, 9, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((cu[-1], hq, d))
    k = rng.standard_normal((cu[-1], hkv, d))
    v = rng.standard_normal((cu[-1], hkv, d))
    do = rng.standard_normal((cu[-1], hq, d))
    o, l = oracle.attention_varlen_ref(q, k, v, cu, cu, causal=True, alibi_slopes=table)
    dq, dk, dv = oracle.attention_bwd_varlen_ref(q, k, v, do, cu, cu, causal=True, alibi_slopes=table)
    for s_ in range(len(lens)):
        a, z = cu[s_], cu[s_ + 1]
        ro, rl = oracle.attention_ref(q[None, a:z], k[None, a:z], v[None, a:z], causal=True,
                                      alibi_slopes=list(table[s_]))
        assert np.array_equal(o[a:z], ro[0]) and np.array_equal(l[:, a:z], rl[0])
        gq, gk, gv = oracle.attention_bwd_ref(q[None, a:z], k[None, a:z], v[None, a:z],
                                              do[None, a:z], causal=True, alibi_slopes=list(table[s_]))
        assert np.array_equal(dq[a:z], gq[0]) and np.array_equal(dk[a:z], gk[0])
        assert np.array_equal(dv[a:z], gv[0])
    # the rows differ enough that a wrong row is visible
    o_wrong, _ = oracle.attention_ref(q[None, cu[1]:cu[2]], k[None, cu[1]:cu[2]], v[None, cu[1]:cu[2]],
                                      causal=True, alibi_slopes=list(table[0]))
    assert np.max(np.abs(o_wrong[0] - o[cu[1]:cu[2]])) > 1e-3
    # kv-cache: cache entry b, valid length n_b, row b of the table
    sk, nq = 11, 3
    kc = rng.standard_normal((3, sk, hkv, d))
    vc = rng.standard_normal((3, sk, hkv, d))
    qc = rng.standard_normal((3, nq, hq, d))
    n_valid = [11, 5, 8]
    oc, lc = oracle.attention_kvcache_ref(qc, kc, vc, cache_seqlens=n_valid, causal=True,
                                          alibi_slopes=table)
    for b in range(3):
        n = n_valid[b]
        ro, rl = oracle.attention_ref(qc[b:b + 1], kc[b:b + 1, :n], vc[b:b + 1, :n], causal=True,
                                      alibi_slopes=list(table[b]))
        assert np.array_equal(oc[b], ro[0]) and np.array_equal(lc[b], rl[0])


def _stats_case(rises_log2, block_k=2):
    """One query row and one key per tile position: tile i holds a key of score u_i (natural
    units, scale 1) and a key 40 nats lower, with u_i the running sum of rises_log2 times ln 2."""
    ln2 = math.log(2.0)
    u = np.cumsum([0.0] + list(rises_log2)) * ln2
    n = len(u)
    q = np.zeros((1, 1, 1, 2)); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, n * block_k, 1, 2))
    for i, ui in enumerate(u):
        k[0, i * block_k, 0, 0] = ui
        for j in range(1, block_k):
            k[0, i * block_k + j, 0, 0] = ui - 40.0
    v = np.ones((1, n * block_k, 1, 2))
    return q, k, v


def pin_tiled_row_stats():
    """Per-row counts of the threshold rule on tiles whose maxima rise by known amounts (log2
    units): rises 3, 6, 0.5, 11, -1 from a first tile at 0 give, at tau = 8, first, skip (3 <= 8,
    max stays at 0), rescale (cumulative 9 > 8, max 9), skip (0.5), rescale (11), skip (-1);
    the largest P is 2^3 = 8, formed on the second tile while the max lags at 0.  A rise of
    exactly 8 is skipped and gives P = 256 ([v1.7] section 1.2).  At tau = 0 every rise
    rescales.  first + skips + rescales = live tiles, counted from the mask in closed form."""
    q, k, v = _stats_case([3, 6, 0.5, 11, -1])
    *_, rs = oracle.tiled_ref(q, k, v, scale=1.0, tau=8.0, block_k=2, return_row_stats=True)
    assert (rs["first"][0, 0, 0], rs["skips"][0, 0, 0], rs["rescales"][0, 0, 0]) == (1, 3, 2)
    assert abs(rs["max_p"][0, 0, 0] - 8.0) < 1e-12
    *_, rs = oracle.tiled_ref(q, k, v, scale=1.0, tau=0.0, block_k=2, return_row_stats=True)
    assert (rs["first"][0, 0, 0], rs["skips"][0, 0, 0], rs["rescales"][0, 0, 0]) == (1, 1, 4)
    assert abs(rs["max_p"][0, 0, 0] - 1.0) < 1e-12
    q, k, v = _stats_case([8.0])
    *_, rs = oracle.tiled_ref(q, k, v, scale=1.0, tau=8.0, block_k=2, return_row_stats=True)
    assert (rs["first"][0, 0, 0], rs["skips"][0, 0, 0], rs["rescales"][0, 0, 0]) == (1, 1, 0)
    assert abs(rs["max_p"][0, 0, 0] - 256.0) < 1e-9
    # live-tile identity on a causal window problem with Sq != Sk and empty rows
    rng = _rng(42)
    sq, sk, bk, wl = 37, 53, 8, 5
    qq = rng.standard_normal((1, sq, 2, 8))
    kk = rng.standard_normal((1, sk, 1, 8)) * (1.0 + np.arange(sk) / 10.0)[None, :, None, None]
    vv = rng.standard_normal((1, sk, 1, 8))
    for kw in (dict(causal=True, window=(wl, -1)), dict(causal=False, window=(3, 0)),
               dict(causal=True, window=(-1, -1))):
        *_, rs = oracle.tiled_ref(qq, kk, vv, tau=8.0, block_k=bk, return_row_stats=True, **kw)
        for i in range(sq):
            n, lo, hi = _visible_count(i, sq, sk, kw["causal"], *kw["window"])
            tiles = 0 if n == 0 else hi // bk - lo // bk + 1
            tot = rs["first"][0, :, i] + rs["skips"][0, :, i] + rs["rescales"][0, :, i]
            assert np.all(tot == tiles), (kw, i)
            assert np.all(rs["first"][0, :, i] == (1 if n else 0))
            assert np.all(rs["max_p"][0, :, i] <= 256.0 + 1e-9)


ALL_PINS = [
    pin_uniform_scores,
    pin_one_hot_scores,
    pin_softcap_single_key,
    pin_rows_sum_to_one,
    pin_permutation_invariance,
    pin_bruteforce_tiny,
    pin_lse_reconstructs_output,
    pin_page_window_00_is_v,
    pin_page_single_row_and_causal_row0,
    pin_page_lse_units,
    pin_decode_is_last_prefill_row,
    pin_paged_cache_is_contiguous,
    pin_alibi_closed_forms,
    pin_alibi_after_softcap,
    pin_alibi_sdpa,
    pin_bwd_autograd,
    pin_bwd_finite_differences,
    pin_bwd_invariants,
    pin_bwd_varlen_is_per_sequence,
    pin_torch_sdpa,
    pin_varlen_block_diagonal,
    pin_gqa_is_repeated_mha,
    pin_tiled_equals_definition,
    pin_page_threshold_numbers,
    pin_nonlagging_is_wrong_at_tau8,
    pin_p_bound,
    pin_bf16_rounding_helper,
    pin_metrics,
    pin_gates_are_the_pages,
    pin_cosine_hand_values,
    pin_compare_each_gate,
    pin_alibi_per_sequence_slopes,
    pin_tiled_row_stats,
]
