"""Tensors whose data lies more than 2 GiB past their base address.

Element offsets are formed in 64 bits (batch, token and page strides times their indices), and
only the offsets within one tile are 32-bit.  These cases put a batch entry, a packed sequence or
a cache row more than 2^31 bytes from the start of its buffer and compare the result there with
the oracle.  Every buffer is NaN-filled outside the valid data: a read that strays into it shows
up as a NaN in the output, and the gap between two batch entries must still be NaN after the
call (no write strayed either); the packed varlen tensors are all data.  The inputs are small
where it counts (a few hundred live rows), so the oracle runs on compact copies.
"""

import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from gpu_common import gate_check, gpu_required, np64

pytestmark = pytest.mark.gpu

GAP = (1 << 31) + 4096  # bytes between batch entries: entry 1 starts past 2 GiB


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gpu_required()
    yield
    torch.cuda.empty_cache()


def _eng():
    import exact_tiled_attention_fa2_amd as eng
    return eng


def _far(shape, dtype, src=None):
    """A [B, S, H, D] view into a NaN-filled buffer with GAP bytes between batch entries (rows,
    heads and dims packed as usual); src, if given, is copied in.  Returns (buffer, view)."""
    b, s, h, d = shape
    row = h * d
    bstride = GAP // 2
    buf = torch.full(((b - 1) * bstride + s * row,), float("nan"), dtype=dtype, device="cuda")
    view = buf.as_strided(shape, (bstride, row, d, 1))
    if src is not None:
        view.copy_(src)
    return buf, view


def _gap_is_nan(buf, shape):
    b, s, h, d = shape
    used = s * h * d
    for i in range(b - 1):
        gap = buf[i * (GAP // 2) + used:(i + 1) * (GAP // 2)]
        assert torch.isnan(gap).all(), "a write strayed into the gap between batch entries"


def _np_contig(t):
    return np64(t.contiguous())


@pytest.mark.parametrize("d,dtype,kw", [(128, "bf16", dict(causal=True)),
                                        (256, "fp16", dict(causal=True, softcap=30.0))])
def test_fwd_batch_entry_past_2gib(d, dtype, kw):
    print(f"[case] fwd far batch entry D={d} {dtype} {kw}", flush=True)
    eng = _eng()
    shape_q, shape_kv = (2, 300, 8, d), (2, 300, 2, d)
    q0, k0, v0 = W.make_dense(400 + d, 2, 300, 300, 8, 2, d, dtype, device="cuda")
    _, q = _far(shape_q, q0.dtype, q0)
    _, k = _far(shape_kv, k0.dtype, k0)
    _, v = _far(shape_kv, v0.dtype, v0)
    obuf, o = _far(shape_q, q0.dtype)
    _, lse = eng.attn_fwd(q, k, v, out=o, **kw)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_ref(np64(q0), np64(k0), np64(v0), causal=kw.get("causal", False),
                                  softcap=kw.get("softcap", 0.0))
    gate_check(_np_contig(o), ro, np64(lse), rl, dtype, f"far fwd D={d}")
    _gap_is_nan(obuf, shape_q)


def test_bwd_batch_entry_past_2gib():
    print("[case] bwd far batch entry D=128 bf16 causal", flush=True)
    eng = _eng()
    shape_q, shape_kv = (2, 260, 8, 128), (2, 260, 2, 128)
    q0, k0, v0 = W.make_dense(410, 2, 260, 260, 8, 2, 128, "bf16", device="cuda")
    do0 = W.randn16(shape_q, "bf16", W._gen(411, "cuda"), "cuda")
    _, q = _far(shape_q, q0.dtype, q0)
    _, k = _far(shape_kv, k0.dtype, k0)
    _, v = _far(shape_kv, v0.dtype, v0)
    _, do = _far(shape_q, q0.dtype, do0)
    _, o = _far(shape_q, q0.dtype)
    _, lse = eng.attn_fwd(q, k, v, out=o, causal=True)
    dqb, dq = _far(shape_q, q0.dtype)
    dkb, dk = _far(shape_kv, q0.dtype)
    dvb, dv = _far(shape_kv, q0.dtype)
    eng.attn_bwd(q, k, v, o, lse, do, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd_ref(np64(q0), np64(k0), np64(v0), np64(do0), causal=True)
    for name, got, ref in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        res = oracle.compare(_np_contig(got), ref, dtype="bf16")
        print(f"[parity] far bwd {name}: {res}", flush=True)
        assert res["finite"] and res["rel_linf"] <= 4e-2 and res["cosine"] >= 0.9995, (name, res)
    _gap_is_nan(dqb, shape_q)
    _gap_is_nan(dkb, shape_kv)
    _gap_is_nan(dvb, shape_kv)


def test_kvcache_rows_past_2gib():
    """B=9 caches of 2^20 tokens x 1 KV head x D=128 (2.25 GiB each): entry 8 starts at 2 GiB."""
    print("[case] kvcache far rows B=9 Sk=2^20 bf16", flush=True)
    eng = _eng()
    b, cap, hq, hkv, d = 9, 1 << 20, 4, 1, 128
    g = torch.Generator(device="cpu").manual_seed(420)
    lens = torch.randint(1, 4097, (b,), generator=g)
    lens[-1] = 4096
    kc = torch.full((b, cap, hkv, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    q, kv_k, kv_v, _ = W.make_kvcache(421, b, 1, 4096, hq, hkv, d, "bf16", device="cuda")
    for i in range(b):
        n = int(lens[i])
        kc[i, :n] = kv_k[i, :n]
        vc[i, :n] = kv_v[i, :n]
    lens_d = lens.to(torch.int32).cuda()
    o, lse = eng.attn_fwd_kvcache(q, kc, vc, cache_seqlens=lens_d, num_splits=16, causal=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_kvcache_ref(np64(q), np64(kc[:, :4096]), np64(vc[:, :4096]),
                                          lens.numpy(), causal=True)
    gate_check(np64(o), ro, np64(lse), rl, "bf16", "far kvcache")


def test_varlen_sequences_past_2gib():
    """Packed q/k/v of ~280k tokens x 32 heads x D=128 (2.2 GB each): the last two sequences lie
    past 2 GiB in every tensor.  The first two are cheap (270,000 queries against one key, one
    query against 270,000 keys), the last two are checked against the oracle; the first one's
    rows, each seeing one key, must equal that key's V row exactly."""
    print("[case] varlen far sequences 32 heads D=128 bf16", flush=True)
    eng = _eng()
    h, d = 32, 128
    lq = [270000, 1, 100, 257]
    lk = [1, 270000, 300, 129]
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    assert int(cq[2]) * h * d * 2 > (1 << 31) and int(ck[2]) * h * d * 2 > (1 << 31)
    gen = W._gen(430, "cuda")
    q = W.randn16((int(cq[-1]), h, d), "bf16", gen, "cuda")
    k = W.randn16((int(ck[-1]), h, d), "bf16", gen, "cuda")
    v = W.randn16((int(ck[-1]), h, d), "bf16", gen, "cuda")
    cu_q = torch.tensor(cq, device="cuda")
    cu_k = torch.tensor(ck, device="cuda")
    o, lse = eng.attn_fwd_varlen(q, k, v, cu_q, cu_k, max(lq), max(lk), causal=False)
    torch.cuda.synchronize()
    # sequence 0: every row sees its one key, so O is that key's V row, bit for bit
    assert torch.equal(o[: lq[0]].view(torch.int16), v[0:1].expand(lq[0], h, d).view(torch.int16))
    for s in (2, 3):
        qs, ks = slice(int(cq[s]), int(cq[s + 1])), slice(int(ck[s]), int(ck[s + 1]))
        ro, rl = oracle.attention_ref(np64(q[qs])[None], np64(k[ks])[None], np64(v[ks])[None])
        gate_check(np64(o[qs])[None], ro, np64(lse[:, qs])[None], rl, "bf16", f"far varlen seq {s}")
