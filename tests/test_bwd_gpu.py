"""GPU parity of the backward (attn_bwd, attn_bwd_varlen) against the fp64 CPU oracle.

The HIP path runs its own forward (attn_fwd) for O and LSE and then its
backward; the oracle computes the gradients from Q, K, V and dO alone.  Every
input is seeded and synthetic.  Gates (rel_Linf = max |g - g_ref| / max
|g_ref| per gradient tensor, cosine over the tensor) are derived from the
arithmetic: P and dS enter the MFMAs rounded to the 16-bit input type, O is
16-bit in D = rowsum(dO * O), and the gradients are stored in 16 bits -- a
few roundings of unit roundoff u (2^-8 bf16, 2^-11 fp16) per element, so
rel_Linf <= 10 u and 1 - cosine <= 1e-4 (bf16) / 1e-5 (fp16).  A gradient
whose exact value is zero everywhere (window (0, 0): P = 1 on the diagonal
makes dT = P (dP - D) vanish) is held to an absolute bound instead.
"""

import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from gpu_common import force_variants, gpu_required, nan_like, np64, run_jobs

pytestmark = pytest.mark.gpu

# rel_Linf and cosine gates per dtype (see the module docstring).
BWD_GATES = {"fp16": (5e-3, 0.99999), "bf16": (4e-2, 0.9999)}
ZERO_REF_ABS = 1e-4   # |g| bound where the exact gradient is 0 (inputs are O(1))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gpu_required()


def _eng():
    import exact_tiled_attention_fa2_amd as eng
    return eng


def grad_check(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    if np.max(np.abs(ref)) < 1e-12:
        mx = float(np.max(np.abs(got)))
        print(f"[parity] {what}: exact gradient is 0, max |g| = {mx:.3e}", flush=True)
        assert np.all(np.isfinite(got)) and mx <= ZERO_REF_ABS, f"{what}: {mx}"
        return
    rl = oracle.rel_linf(got, ref)
    cs = oracle.cosine(got, ref)
    fin = bool(np.all(np.isfinite(got)))
    print(f"[parity] {what}: rel_linf={rl:.3e} cosine={cs:.7f} max_abs={np.max(np.abs(got - ref)):.3e}",
          flush=True)
    rel_gate, cos_gate = BWD_GATES[dtype]
    assert fin, f"{what}: non-finite gradient"
    assert rl <= rel_gate and cs >= cos_gate, f"{what}: rel_linf {rl} cosine {cs}"


def _dout(seed, shape, dtype):
    g = torch.Generator(device="cuda").manual_seed(seed + 7777)
    return W.randn16(shape, dtype, g, device="cuda")


def _opts_np(kw):
    out = dict(kw)
    if out.get("alibi_slopes") is not None:
        out["alibi_slopes"] = out["alibi_slopes"].cpu().numpy().astype(np.float64)
    return out


DENSE = [
    # seed, b, sq, sk, hq, hkv, d, dtype, options
    (81, 1, 200, 200, 4, 4, 128, "fp16", dict(causal=True)),
    (82, 2, 300, 300, 8, 2, 128, "bf16", dict(causal=True)),
    (83, 1, 130, 333, 4, 2, 64, "fp16", dict(causal=False)),
    (84, 1, 257, 257, 4, 1, 128, "bf16", dict(causal=True, window=(64, 0), softcap=30.0)),
    (85, 2, 190, 190, 4, 4, 64, "fp16", dict(causal=True, alibi=True)),
    (86, 1, 300, 100, 2, 2, 128, "bf16", dict(causal=True)),          # rows with no key
    (87, 1, 64, 64, 2, 1, 128, "fp16", dict(causal=False, window=(0, 0))),
    (88, 2, 97, 161, 6, 3, 64, "bf16", dict(causal=False, softcap=5.0, alibi=True)),
    # ALiBi over many steps whose query head changes within a dK/dV walk (the slope of the next
    # step is loaded one step ahead)
    (89, 1, 700, 700, 8, 2, 128, "bf16", dict(causal=True, alibi=True)),
    # head_dim 256 (32-query steps in the paired dK/dV kernel; dQ at one wave per SIMD)
    (181, 1, 257, 257, 4, 2, 256, "fp16", dict(causal=True)),
    (182, 2, 190, 300, 4, 1, 256, "bf16", dict(causal=False, softcap=20.0, alibi=True)),
    (183, 1, 300, 200, 2, 2, 256, "fp16", dict(causal=True, window=(64, 0))),   # rows with no key
    # long walks at head_dim 256 (K / V fragments partly in LDS) with every score transform
    (184, 1, 1100, 1100, 8, 2, 256, "bf16", dict(causal=True, softcap=30.0, alibi=True)),
    (185, 1, 900, 1300, 4, 4, 256, "fp16", dict(causal=False, alibi=True)),
]


@pytest.mark.parametrize("case", DENSE, ids=[f"s{c[0]}" for c in DENSE])
def test_bwd_dense(case):
    seed, b, sq, sk, hq, hkv, d, dtype, kw = case
    kw = dict(kw)
    print(f"[case] bwd dense seed={seed} b={b} sq={sq} sk={sk} hq={hq} hkv={hkv} d={d} {dtype} {kw}", flush=True)
    if kw.pop("alibi", False):
        kw["alibi_slopes"] = W.alibi_slopes(hq, b, device="cuda")
    eng = _eng()
    q, k, v = W.make_dense(seed, b, sq, sk, hq, hkv, d, dtype, device="cuda")
    do = _dout(seed, (b, sq, hq, d), dtype)
    o, lse = eng.attn_fwd(q, k, v, **kw)
    dq, dk, dv = eng.attn_bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd_ref(np64(q), np64(k), np64(v), np64(do), **_opts_np(kw))
    grad_check(np64(dq), rq, dtype, f"dQ {seed}")
    grad_check(np64(dk), rk, dtype, f"dK {seed}")
    grad_check(np64(dv), rv, dtype, f"dV {seed}")
    if sq > sk and kw.get("causal"):
        assert torch.all(dq[:, : sq - sk] == 0)


def test_bwd_varlen():
    """Packed sequences (one of length 1, one empty), GQA, causal."""
    print("[case] bwd varlen", flush=True)
    eng = _eng()
    lens = [100, 1, 0, 257, 64]
    q, k, v, cu, lens = W.make_varlen(89, len(lens), 1, 1, 8, 2, 128, "bf16", device="cuda", lengths=lens)
    do = _dout(89, tuple(q.shape), "bf16")
    o, lse = eng.attn_fwd_varlen(q, k, v, cu, cu, max(lens), max(lens), causal=True)
    dq, dk, dv = eng.attn_bwd_varlen(q, k, v, o, lse, do, cu, cu, max(lens), max(lens), causal=True)
    torch.cuda.synchronize()
    cu_np = cu.cpu().numpy()
    rq, rk, rv = oracle.attention_bwd_varlen_ref(np64(q), np64(k), np64(v), np64(do), cu_np, cu_np, causal=True)
    grad_check(np64(dq), rq, "bf16", "varlen dQ")
    grad_check(np64(dk), rk, "bf16", "varlen dK")
    grad_check(np64(dv), rv, "bf16", "varlen dV")


@pytest.mark.parametrize("case", [(185, 64, "fp16", dict(causal=True, window=(48, 0), softcap=10.0)),
                                  (186, 128, "bf16", dict(causal=False, window=(80, 40)))],
                         ids=["s185", "s186"])
def test_bwd_varlen_alibi(case):
    """Packed sequences (one of length 1, one empty) with per-sequence ALiBi slopes [B, Hq], GQA,
    and a window (with softcap, or non-causal with both bounds)."""
    seed, d, dtype, kw = case
    print(f"[case] bwd varlen alibi seed={seed} d={d} {dtype} {kw}", flush=True)
    eng = _eng()
    lens = [90, 1, 0, 211, 47]
    q, k, v, cu, lens = W.make_varlen(seed, len(lens), 1, 1, 8, 2, d, dtype, device="cuda", lengths=lens)
    sl = W.alibi_slopes(8, len(lens), device="cuda")
    do = _dout(seed, tuple(q.shape), dtype)
    o, lse = eng.attn_fwd_varlen(q, k, v, cu, cu, max(lens), max(lens), alibi_slopes=sl, **kw)
    dq, dk, dv = eng.attn_bwd_varlen(q, k, v, o, lse, do, cu, cu, max(lens), max(lens), alibi_slopes=sl, **kw)
    torch.cuda.synchronize()
    cu_np = cu.cpu().numpy()
    rq, rk, rv = oracle.attention_bwd_varlen_ref(np64(q), np64(k), np64(v), np64(do), cu_np, cu_np,
                                                 alibi_slopes=np64(sl), **kw)
    grad_check(np64(dq), rq, dtype, f"varlen alibi {seed} dQ")
    grad_check(np64(dk), rk, dtype, f"varlen alibi {seed} dK")
    grad_check(np64(dv), rv, dtype, f"varlen alibi {seed} dV")


def test_bwd_varlen_d256():
    """Packed sequences at head_dim 256 (one of length 1, one empty), GQA, causal, fp16."""
    print("[case] bwd varlen d256", flush=True)
    eng = _eng()
    lens = [130, 1, 0, 200, 33]
    q, k, v, cu, lens = W.make_varlen(184, len(lens), 1, 1, 8, 2, 256, "fp16", device="cuda", lengths=lens)
    do = _dout(184, tuple(q.shape), "fp16")
    o, lse = eng.attn_fwd_varlen(q, k, v, cu, cu, max(lens), max(lens), causal=True)
    dq, dk, dv = eng.attn_bwd_varlen(q, k, v, o, lse, do, cu, cu, max(lens), max(lens), causal=True)
    torch.cuda.synchronize()
    cu_np = cu.cpu().numpy()
    rq, rk, rv = oracle.attention_bwd_varlen_ref(np64(q), np64(k), np64(v), np64(do), cu_np, cu_np, causal=True)
    grad_check(np64(dq), rq, "fp16", "varlen d256 dQ")
    grad_check(np64(dk), rk, "fp16", "varlen d256 dK")
    grad_check(np64(dv), rv, "fp16", "varlen d256 dV")


def test_bwd_cfg5b_shape_whole():
    """The backward at the fp16 D=256 prefill shape (B=4, Sq=Sk=4096, 32 query / 8 KV heads,
    causal) against the oracle on the whole dQ, dK and dV (dK, dV sum their four query heads);
    the gradients start as NaN so an unwritten tile fails."""
    print("[case] bwd cfg5b shape whole", flush=True)
    eng = _eng()
    c = W.WORKLOADS["cfg5b_fp16_d256_causal"]
    b_, s, hq, hkv, d = c["batch"], c["seqlen_q"], c["heads_q"], c["heads_kv"], c["head_dim"]
    q, k, v = W.make_dense(c["seed"], b_, s, s, hq, hkv, d, c["dtype"], device="cuda")
    do = _dout(c["seed"], tuple(q.shape), c["dtype"])
    o, lse = eng.attn_fwd(q, k, v, causal=True)
    dq, dk, dv = nan_like(q), nan_like(k), nan_like(v)
    eng.attn_bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    qn, kn, vn, don = np64(q), np64(k), np64(v), np64(do)
    g = hq // hkv

    def ref(job):
        bi, kh = job
        hs = slice(kh * g, (kh + 1) * g)
        return oracle.attention_bwd_ref(np.ascontiguousarray(qn[bi:bi + 1, :, hs]),
                                        np.ascontiguousarray(kn[bi:bi + 1, :, kh:kh + 1]),
                                        np.ascontiguousarray(vn[bi:bi + 1, :, kh:kh + 1]),
                                        np.ascontiguousarray(don[bi:bi + 1, :, hs]), causal=True)

    jobs = [(bi, kh) for bi in range(b_) for kh in range(hkv)]
    rq, rk, rv = np.empty(qn.shape), np.empty(kn.shape), np.empty(vn.shape)
    for (bi, kh), (gq, gk, gv) in zip(jobs, run_jobs(ref, jobs)):
        rq[bi, :, kh * g:(kh + 1) * g] = gq[0]
        rk[bi, :, kh], rv[bi, :, kh] = gk[0, :, 0], gv[0, :, 0]
    del qn, kn, vn, don
    grad_check(np64(dq), rq, "fp16", "cfg5b shape dQ")
    grad_check(np64(dk), rk, "fp16", "cfg5b shape dK")
    grad_check(np64(dv), rv, "fp16", "cfg5b shape dV")


def test_bwd_deterministic():
    """No atomics: two calls give the same bits."""
    print("[case] bwd determinism", flush=True)
    eng = _eng()
    q, k, v = W.make_dense(90, 2, 333, 333, 8, 2, 128, "bf16", device="cuda")
    do = _dout(90, tuple(q.shape), "bf16")
    o, lse = eng.attn_fwd(q, k, v, causal=True)
    g1 = eng.attn_bwd(q, k, v, o, lse, do, causal=True)
    g2 = eng.attn_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for a, c in zip(g1, g2):
        assert torch.equal(a, c)


def test_bwd_pages_gradient_check():
    """The pages' backward check: fp16, S = 1024, causal, gradients against a high-precision
    reference (here the fp64 oracle); all four (batch, head) pairs in full."""
    print("[case] bwd fp16 1024 causal", flush=True)
    eng = _eng()
    b, s, h, d = 2, 1024, 2, 128
    q, k, v = W.make_dense(91, b, s, s, h, h, d, "fp16", device="cuda")
    do = _dout(91, (b, s, h, d), "fp16")
    o, lse = eng.attn_fwd(q, k, v, causal=True)
    dq, dk, dv = eng.attn_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd_ref(np64(q), np64(k), np64(v), np64(do), causal=True)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        grad_check(np64(g), r, "fp16", f"1024 {name}")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_bwd_finite_2k(dtype):
    """The pages' finiteness probe: S = 2048, causal, both dtypes: every gradient finite."""
    print(f"[case] bwd finite 2048 {dtype}", flush=True)
    eng = _eng()
    q, k, v = W.make_dense(92, 2, 2048, 2048, 8, 8, 128, dtype, device="cuda")
    do = _dout(92, tuple(q.shape), dtype)
    o, lse = eng.attn_fwd(q, k, v, causal=True)
    for g in eng.attn_bwd(q, k, v, o, lse, do, causal=True):
        assert torch.isfinite(g).all()


@pytest.mark.parametrize("variant", ["1", "2", "3", "4"])
def test_bwd_variants(variant, request):
    """The debug build's kernel shapes (two-pass dK/dV; dQ with 256 / 128 queries per workgroup;
    one-pass dK/dV at one wave per SIMD) on a ragged GQA causal case with a window and softcap."""
    force_variants(request, bwd=int(variant))
    print(f"[case] bwd variant {variant}", flush=True)
    eng = _eng()
    kw = dict(causal=True, window=(100, 0), softcap=20.0)
    q, k, v = W.make_dense(93, 2, 333, 333, 4, 2, 128, "bf16", device="cuda")
    do = _dout(93, tuple(q.shape), "bf16")
    o, lse = eng.attn_fwd(q, k, v, **kw)
    dq, dk, dv = eng.attn_bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd_ref(np64(q), np64(k), np64(v), np64(do), **kw)
    grad_check(np64(dq), rq, "bf16", f"variant {variant} dQ")
    grad_check(np64(dk), rk, "bf16", f"variant {variant} dK")
    grad_check(np64(dv), rv, "bf16", f"variant {variant} dV")


D256 = [c for c in DENSE if c[6] == 256]


@pytest.mark.parametrize("case", D256, ids=[f"s{c[0]}" for c in D256])
def test_bwd_d256_two_walk_variant(case, request):
    """dK/dV in two walks at one wave per SIMD (debug override 4 at head_dim 256: dV from S and P,
    then dK from S, dP and dS) on the D = 256 cases."""
    force_variants(request, bwd=4)
    seed, b, sq, sk, hq, hkv, d, dtype, kw = case
    kw = dict(kw)
    print(f"[case] bwd d256 two-walk seed={seed} b={b} sq={sq} sk={sk} hq={hq} hkv={hkv} {dtype} {kw}", flush=True)
    if kw.pop("alibi", False):
        kw["alibi_slopes"] = W.alibi_slopes(hq, b, device="cuda")
    eng = _eng()
    q, k, v = W.make_dense(seed, b, sq, sk, hq, hkv, d, dtype, device="cuda")
    do = _dout(seed, (b, sq, hq, d), dtype)
    o, lse = eng.attn_fwd(q, k, v, **kw)
    dq, dk, dv = eng.attn_bwd(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd_ref(np64(q), np64(k), np64(v), np64(do), **_opts_np(kw))
    grad_check(np64(dq), rq, dtype, f"two-walk d256 dQ {seed}")
    grad_check(np64(dk), rk, dtype, f"two-walk d256 dK {seed}")
    grad_check(np64(dv), rv, dtype, f"two-walk d256 dV {seed}")


def test_bwd_headline_whole():
    """The benchmarked backward shape (bf16, B=4, Sq=Sk=2048, 16 heads, D=128, causal) in its default
    launch configuration (256-query dQ tiles), against the oracle on the whole dQ, dK and dV; the
    gradients start as NaN so an unwritten tile fails."""
    print("[case] bwd headline whole", flush=True)
    eng = _eng()
    c = W.WORKLOADS["bwd_cfg2_bf16_causal_2k"]
    b_, s, h_, d = c["batch"], c["seqlen_q"], c["heads_q"], c["head_dim"]
    q, k, v = W.make_dense(c["seed"], b_, s, s, h_, h_, d, c["dtype"], device="cuda")
    do = _dout(c["seed"], tuple(q.shape), c["dtype"])
    o, lse = eng.attn_fwd(q, k, v, causal=True)
    dq, dk, dv = nan_like(q), nan_like(k), nan_like(v)
    eng.attn_bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    qn, kn, vn, don = np64(q), np64(k), np64(v), np64(do)

    def ref(job):
        bi, hi = job
        sl = (slice(bi, bi + 1), slice(None), slice(hi, hi + 1))
        return oracle.attention_bwd_ref(np.ascontiguousarray(qn[sl]), np.ascontiguousarray(kn[sl]),
                                        np.ascontiguousarray(vn[sl]), np.ascontiguousarray(don[sl]),
                                        causal=True)

    jobs = [(bi, hi) for bi in range(b_) for hi in range(h_)]
    rq, rk, rv = np.empty(qn.shape), np.empty(kn.shape), np.empty(vn.shape)
    for (bi, hi), (gq, gk, gv) in zip(jobs, run_jobs(ref, jobs)):
        rq[bi, :, hi], rk[bi, :, hi], rv[bi, :, hi] = gq[0, :, 0], gk[0, :, 0], gv[0, :, 0]
    grad_check(np64(dq), rq, c["dtype"], "headline dQ")
    grad_check(np64(dk), rk, c["dtype"], "headline dK")
    grad_check(np64(dv), rv, c["dtype"], "headline dV")
