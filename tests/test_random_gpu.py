"""GPU parity on seeded random problems: every feature of the forward and the backward in random
combination (dtype, head dim, GQA group, lengths including 1 and Sq != Sk, causal, window,
softcap, ALiBi) and under each selectable tile shape, against the fp64 oracle on the whole
output.  The draws are fixed by the seeds below, so a failure names a reproducible case.
"""

import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from gpu_common import force_variants, gate_check, gpu_required, np64

pytestmark = pytest.mark.gpu

# rel_Linf and cosine gates of the backward per dtype (as in the backward parity tests).
BWD_GATES = {"fp16": (5e-3, 0.99999), "bf16": (4e-2, 0.9999)}
ZERO_REF_ABS = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gpu_required()


def _eng():
    import exact_tiled_attention_fa2_amd as eng
    return eng


def _draw(seed, head_dims):
    """One random problem: shapes, options and the forward tile variant to force."""
    rng = np.random.default_rng(seed)
    d = int(rng.choice(head_dims))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4]))
    sq = int(rng.choice([1, int(rng.integers(2, 80)), int(rng.integers(80, 600))]))
    sk = sq if rng.random() < 0.5 else int(rng.integers(1, 600))
    kw = dict(causal=bool(rng.random() < 0.6))
    if rng.random() < 0.3:
        kw["window"] = (int(rng.integers(0, 200)), int(rng.integers(0, 50)) if not kw["causal"] else 0)
    if rng.random() < 0.3:
        kw["softcap"] = float(rng.choice([5.0, 30.0]))
    alibi = bool(rng.random() < 0.25)
    return dict(seed=seed, b=int(rng.integers(1, 4)), sq=sq, sk=sk, hq=hkv * g, hkv=hkv, d=d,
                dtype=str(rng.choice(["bf16", "fp16"])), kw=kw, alibi=alibi,
                variant=str(rng.choice(["0", "1", "2", "5"])))


FWD_SEEDS = list(range(5000, 5036))
BWD_SEEDS = list(range(6000, 6012))
BWD_SEEDS_D256 = list(range(6100, 6106))


@pytest.mark.parametrize("seed", FWD_SEEDS)
def test_random_forward(seed, request):
    c = _draw(seed, [64, 128, 256])
    force_variants(request, fwd=int(c["variant"]))
    print(f"[case] random forward {c}", flush=True)
    kw = dict(c["kw"])
    if c["alibi"]:
        kw["alibi_slopes"] = W.alibi_slopes(c["hq"], c["b"], device="cuda")
    q, k, v = W.make_dense(seed, c["b"], c["sq"], c["sk"], c["hq"], c["hkv"], c["d"], c["dtype"], device="cuda")
    o, lse = _eng().attn_fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    ref_kw = dict(kw)
    if c["alibi"]:
        ref_kw["alibi_slopes"] = np64(kw["alibi_slopes"])
    ro, rl = oracle.attention_ref(np64(q), np64(k), np64(v), **ref_kw)
    gate_check(np64(o), ro, np64(lse), rl, c["dtype"], f"random forward {seed}")


def _grad_check(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    if np.max(np.abs(ref)) < 1e-12:
        mx = float(np.max(np.abs(got)))
        print(f"[parity] {what}: exact gradient is 0, max |g| = {mx:.3e}", flush=True)
        assert np.all(np.isfinite(got)) and mx <= ZERO_REF_ABS, f"{what}: {mx}"
        return
    rl, cs = oracle.rel_linf(got, ref), oracle.cosine(got, ref)
    print(f"[parity] {what}: rel_linf={rl:.3e} cosine={cs:.7f}", flush=True)
    rel_gate, cos_gate = BWD_GATES[dtype]
    assert np.all(np.isfinite(got)) and rl <= rel_gate and cs >= cos_gate, f"{what}: {rl} {cs}"


@pytest.mark.parametrize("seed", BWD_SEEDS + BWD_SEEDS_D256)
def test_random_backward(seed, request):
    c = _draw(seed, [256] if seed in BWD_SEEDS_D256 else [64, 128])
    # head_dim 256 has one override (4: the two-walk dK/dV kernel); 64 / 128 have 1-3
    choices = ["0", "4"] if c["d"] == 256 else ["0", "1", "2", "3"]
    bwd_variant = str(np.random.default_rng(seed + 1).choice(choices))
    force_variants(request, bwd=int(bwd_variant))
    print(f"[case] random backward {c} bwd_variant={bwd_variant}", flush=True)
    kw = dict(c["kw"])
    if c["alibi"]:
        kw["alibi_slopes"] = W.alibi_slopes(c["hq"], c["b"], device="cuda")
    eng = _eng()
    q, k, v = W.make_dense(seed, c["b"], c["sq"], c["sk"], c["hq"], c["hkv"], c["d"], c["dtype"], device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(seed + 7777)
    do = W.randn16(tuple(q.shape), c["dtype"], gen, device="cuda")
    o, lse = eng.attn_fwd(q, k, v, **kw)
    dq, dk, dv = eng.attn_bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    ref_kw = dict(kw)
    if c["alibi"]:
        ref_kw["alibi_slopes"] = np64(kw["alibi_slopes"])
    rq, rk, rv = oracle.attention_bwd_ref(np64(q), np64(k), np64(v), np64(do), **ref_kw)
    _grad_check(np64(dq), rq, c["dtype"], f"random dQ {seed}")
    _grad_check(np64(dk), rk, c["dtype"], f"random dK {seed}")
    _grad_check(np64(dv), rv, c["dtype"], f"random dV {seed}")


# ------------------------------------------------------------------ packed variable-length problems

def _draw_varlen(seed, head_dims):
    """A random packed batch: 1-6 sequences whose query and key lengths are drawn separately
    (0, 1, short or long; the first sequence has at least one query), and the options of _draw."""
    rng = np.random.default_rng(seed)

    def length():
        u = rng.random()
        return 0 if u < 0.1 else 1 if u < 0.2 else int(rng.integers(2, 100)) if u < 0.5 else int(rng.integers(100, 700))

    n = int(rng.integers(1, 7))
    lq = [length() for _ in range(n)]
    lq[0] = max(lq[0], 1)
    lk = [lq[i] if rng.random() < 0.5 else length() for i in range(n)]
    base = _draw(seed, head_dims)
    return dict(base, lq=lq, lk=lk)


def _varlen_inputs(c):
    cq = np.concatenate([[0], np.cumsum(c["lq"])]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(c["lk"])]).astype(np.int32)
    gen = torch.Generator(device="cuda").manual_seed(c["seed"] + 31)
    q = W.randn16((int(cq[-1]), c["hq"], c["d"]), c["dtype"], gen, device="cuda")
    k = W.randn16((int(ck[-1]), c["hkv"], c["d"]), c["dtype"], gen, device="cuda")
    v = W.randn16((int(ck[-1]), c["hkv"], c["d"]), c["dtype"], gen, device="cuda")
    kw = dict(c["kw"])
    if c["alibi"]:  # per-sequence slopes
        kw["alibi_slopes"] = W.alibi_slopes(c["hq"], len(c["lq"]), device="cuda")
    return q, k, v, torch.tensor(cq, device="cuda"), torch.tensor(ck, device="cuda"), cq, ck, kw


def _np_kw(kw):
    out = dict(kw)
    if out.get("alibi_slopes") is not None:
        out["alibi_slopes"] = np64(out["alibi_slopes"])
    return out


VARLEN_FWD_SEEDS = list(range(5100, 5114)) + [5118, 5119]  # the last four draw head_dim 128
VARLEN_BWD_SEEDS = list(range(6200, 6206)) + [6206, 6208]  # the last two draw head_dim 128


@pytest.mark.parametrize("seed", VARLEN_FWD_SEEDS)
def test_random_varlen_forward(seed, request):
    c = _draw_varlen(seed, [64, 128, 256])
    force_variants(request, fwd=int(c["variant"]))
    print(f"[case] random varlen forward {c}", flush=True)
    q, k, v, cu_q, cu_k, cq, ck, kw = _varlen_inputs(c)
    o, lse = _eng().attn_fwd_varlen(q, k, v, cu_q, cu_k, max(c["lq"]), max(max(c["lk"]), 1), **kw)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_varlen_ref(np64(q), np64(k), np64(v), cq, ck, **_np_kw(kw))
    gate_check(np64(o), ro, np64(lse), rl, c["dtype"], f"random varlen forward {seed}")


@pytest.mark.parametrize("seed", VARLEN_BWD_SEEDS)
def test_random_varlen_backward(seed, request):
    c = _draw_varlen(seed, [64, 128, 256])
    print(f"[case] random varlen backward {c}", flush=True)
    q, k, v, cu_q, cu_k, cq, ck, kw = _varlen_inputs(c)
    eng = _eng()
    mq, mk = max(c["lq"]), max(max(c["lk"]), 1)
    gen = torch.Generator(device="cuda").manual_seed(seed + 7777)
    do = W.randn16(tuple(q.shape), c["dtype"], gen, device="cuda")
    o, lse = eng.attn_fwd_varlen(q, k, v, cu_q, cu_k, mq, mk, **kw)
    dq, dk, dv = eng.attn_bwd_varlen(q, k, v, o, lse, do, cu_q, cu_k, mq, mk, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd_varlen_ref(np64(q), np64(k), np64(v), np64(do), cq, ck, **_np_kw(kw))
    if k.shape[0] == 0:
        assert dk.numel() == 0 and dv.numel() == 0
    _grad_check(np64(dq), rq, c["dtype"], f"random varlen dQ {seed}")
    if k.shape[0] > 0:
        _grad_check(np64(dk), rk, c["dtype"], f"random varlen dK {seed}")
        _grad_check(np64(dv), rv, c["dtype"], f"random varlen dV {seed}")


# ------------------------------------------------------------------ split-KV against a cache

def _draw_kvcache(seed):
    """A random decode or chunked-prefill problem against a cache: random valid lengths with NaN
    past them, contiguous or paged (shuffled pages), a random split count (0 = the heuristic),
    the options of _draw and a random decode tile override."""
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    sq = int(rng.choice([1, 1, 1, int(rng.integers(2, 9)), int(rng.integers(16, 200))]))
    kw = dict(causal=bool(rng.random() < 0.7))
    if rng.random() < 0.3:
        kw["window"] = (int(rng.integers(0, 500)), 0 if kw["causal"] else int(rng.integers(0, 50)))
    if rng.random() < 0.3:
        kw["softcap"] = float(rng.choice([5.0, 30.0]))
    return dict(seed=seed, b=int(rng.integers(1, 5)), sq=sq, sk=int(rng.integers(1, 3000)), hq=hkv * g,
                hkv=hkv, d=d, dtype=str(rng.choice(["bf16", "fp16"])), kw=kw,
                alibi=bool(rng.random() < 0.25), splits=int(rng.choice([0, 1, 2, 3, 5, 8, 16])),
                page=int(rng.choice([0, 0, 64, 128, 256])), dec_variant=int(rng.choice([0, 1, 2])))


KVCACHE_SEEDS = list(range(5300, 5320))


@pytest.mark.parametrize("seed", KVCACHE_SEEDS)
def test_random_kvcache(seed, request):
    c = _draw_kvcache(seed)
    force_variants(request, dec=c["dec_variant"])
    print(f"[case] random kvcache {c}", flush=True)
    eng = _eng()
    q, kc, vc, lens = W.make_kvcache(seed, c["b"], c["sq"], c["sk"], c["hq"], c["hkv"], c["d"], c["dtype"],
                                     device="cuda", random_lengths=True, nan_tail=True)
    kw = dict(c["kw"])
    if c["alibi"]:
        kw["alibi_slopes"] = W.alibi_slopes(c["hq"], c["b"], device="cuda")
    table = None
    if c["page"]:
        kc, vc, table = W.page_cache(kc, vc, lens, c["page"], seed)
    o, lse = eng.attn_fwd_kvcache(q, kc, vc, cache_seqlens=lens, num_splits=c["splits"], block_table=table, **kw)
    torch.cuda.synchronize()
    ref_kw = dict(kw)
    if c["alibi"]:
        ref_kw["alibi_slopes"] = np64(kw["alibi_slopes"])
    ro, rl = oracle.attention_kvcache_ref(np64(q), np64(kc), np64(vc), lens.cpu().numpy(),
                                          block_table=None if table is None else table.cpu().numpy(), **ref_kw)
    gate_check(np64(o), ro, np64(lse), rl, c["dtype"], f"random kvcache {seed}")
