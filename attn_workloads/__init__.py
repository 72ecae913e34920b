"""Seeded synthetic inputs for the attention workloads.

This module is shared by the tests, the smoke check and the benchmark.  It
holds input construction only -- shapes, seeds and value distributions --
and none of the attention arithmetic, so both the GPU path and the CPU
oracle can consume the same tensors without sharing any method code.

Recipe (the pages measure only on synthetic N(0,1)-style tensors):

* values are drawn as fp32 standard normals from a ``torch.Generator``
  seeded with the workload's seed, then rounded to the 16-bit dtype (round
  to nearest even);
* the "K ramp" variant multiplies key row j by
  1 + 3 * floor(j / 128) / (Sk / 128 - 1) in fp32 before rounding, so the
  row max rises from block to block (16 steps from 1.0 to 4.0 at Sk = 2048);
* varlen lengths are drawn uniformly from [lo, hi] with the same generator
  before the tensors, and packed back to back (cu_seqlens = prefix sums);
* decode caches are N(0,1) over the full [B, Sk, Hkv, D] buffer; when
  ``nan_tail`` is set, rows at or beyond each sequence's valid length are
  filled with NaN so that any read of them would show in the output.
"""

import math

import torch

__all__ = [
    "WORKLOADS",
    "DTYPES",
    "randn16",
    "make_dense",
    "make_varlen",
    "make_kvcache",
    "alibi_slopes",
    "k_ramp_factor",
]

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}

# The five workloads the library is measured and checked on, with seeds.
WORKLOADS = {
    "cfg1_fp16_small": dict(kind="dense", seed=1001, batch=1, seqlen_q=128, seqlen_k=128,
                            heads_q=2, heads_kv=2, head_dim=64, dtype="fp16", causal=False,
                            window=(-1, -1), softcap=0.0, scale=1.0 / 8.0),
    "cfg2_bf16_causal_2k": dict(kind="dense", seed=1002, batch=4, seqlen_q=2048, seqlen_k=2048,
                                heads_q=16, heads_kv=16, head_dim=128, dtype="bf16", causal=True,
                                window=(-1, -1), softcap=0.0),
    "cfg2r_bf16_causal_2k_kramp": dict(kind="dense", seed=1002, batch=4, seqlen_q=2048,
                                       seqlen_k=2048, heads_q=16, heads_kv=16, head_dim=128,
                                       dtype="bf16", causal=True, window=(-1, -1), softcap=0.0,
                                       k_ramp=True),
    "cfg3_bf16_varlen": dict(kind="varlen", seed=1003, n_seqs=16, len_lo=64, len_hi=4096,
                             heads_q=32, heads_kv=32, head_dim=128, dtype="bf16", causal=True,
                             window=(-1, -1), softcap=0.0),
    "cfg4_bf16_gqa_window_softcap": dict(kind="dense", seed=1004, batch=2, seqlen_q=8192,
                                         seqlen_k=8192, heads_q=32, heads_kv=8, head_dim=128,
                                         dtype="bf16", causal=True, window=(4096, 0),
                                         softcap=30.0),
    "cfg5a_bf16_decode": dict(kind="kvcache", seed=1005, batch=32, seqlen_q=1, seqlen_k=32768,
                              heads_q=32, heads_kv=8, head_dim=128, dtype="bf16", causal=False,
                              window=(-1, -1), softcap=0.0, num_splits=16),
    "cfg5a_bf16_decode_paged": dict(kind="kvcache", seed=1005, batch=32, seqlen_q=1, seqlen_k=32768,
                                    heads_q=32, heads_kv=8, head_dim=128, dtype="bf16", causal=False,
                                    window=(-1, -1), softcap=0.0, num_splits=16, page=256),
    "cfg2a_bf16_causal_2k_alibi": dict(kind="dense", seed=1002, batch=4, seqlen_q=2048, seqlen_k=2048,
                                       heads_q=16, heads_kv=16, head_dim=128, dtype="bf16", causal=True,
                                       window=(-1, -1), softcap=0.0, alibi=True),
    "cfg5a_bf16_decode_alibi": dict(kind="kvcache", seed=1005, batch=32, seqlen_q=1, seqlen_k=32768,
                                    heads_q=32, heads_kv=8, head_dim=128, dtype="bf16", causal=False,
                                    window=(-1, -1), softcap=0.0, num_splits=16, alibi=True),
    "bwd_cfg2_bf16_causal_2k": dict(kind="bwd", seed=1002, batch=4, seqlen_q=2048, seqlen_k=2048,
                                    heads_q=16, heads_kv=16, head_dim=128, dtype="bf16", causal=True,
                                    window=(-1, -1), softcap=0.0),
    "bwd_fp16_causal_1k": dict(kind="bwd", seed=1007, batch=4, seqlen_q=1024, seqlen_k=1024,
                               heads_q=16, heads_kv=16, head_dim=128, dtype="fp16", causal=True,
                               window=(-1, -1), softcap=0.0),
    "cfg5b_fp16_d256_causal": dict(kind="dense", seed=1006, batch=4, seqlen_q=4096,
                                   seqlen_k=4096, heads_q=32, heads_kv=8, head_dim=256,
                                   dtype="fp16", causal=True, window=(-1, -1), softcap=0.0),
    "bwd_cfg5b_fp16_d256_causal": dict(kind="bwd", seed=1006, batch=4, seqlen_q=4096,
                                       seqlen_k=4096, heads_q=32, heads_kv=8, head_dim=256,
                                       dtype="fp16", causal=True, window=(-1, -1), softcap=0.0),
}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn16(shape, dtype, gen, device="cpu", chunk_elems=1 << 27):
    """N(0,1) fp32 draws rounded to the 16-bit ``dtype`` (filled in chunks to bound memory)."""
    out = torch.empty(shape, dtype=DTYPES.get(dtype, dtype), device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk_elems):
        e = min(s + chunk_elems, flat.numel())
        flat[s:e] = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
    return out


def k_ramp_factor(seqlen_k, granularity=128, device="cpu"):
    """Per-key fp32 multiplier 1 + 3*floor(j/g)/(Sk/g - 1): a ramp from 1 to 4 over key blocks."""
    nblk = max(1, math.ceil(seqlen_k / granularity))
    j = torch.arange(seqlen_k, device=device)
    blk = torch.div(j, granularity, rounding_mode="floor").to(torch.float32)
    return 1.0 + 3.0 * blk / max(1, nblk - 1)


def make_dense(seed, batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim, dtype,
               k_ramp=False, device="cpu", q_scale=1.0):
    """q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D] in the 16-bit dtype, N(0,1) from ``seed``."""
    g = _gen(seed, device)
    q = randn16((batch, seqlen_q, heads_q, head_dim), dtype, g, device)
    if k_ramp:
        k32 = torch.randn((batch, seqlen_k, heads_kv, head_dim), generator=g, device=device,
                          dtype=torch.float32)
        k32 *= k_ramp_factor(seqlen_k, device=device).view(1, seqlen_k, 1, 1)
        k = k32.to(DTYPES[dtype])
        del k32
    else:
        k = randn16((batch, seqlen_k, heads_kv, head_dim), dtype, g, device)
    v = randn16((batch, seqlen_k, heads_kv, head_dim), dtype, g, device)
    if q_scale != 1.0:
        q = (q.to(torch.float32) * q_scale).to(DTYPES[dtype])
    return q, k, v


def make_varlen(seed, n_seqs, len_lo, len_hi, heads_q, heads_kv, head_dim, dtype,
                device="cpu", lengths=None):
    """Packed q [T, Hq, D], k/v [T, Hkv, D] and int32 cu_seqlens [n+1] (q and k share it)."""
    g = _gen(seed, "cpu")
    if lengths is None:
        lengths = torch.randint(len_lo, len_hi + 1, (n_seqs,), generator=g).tolist()
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    total = cu[-1]
    gd = g if device == "cpu" else _gen(seed + 7919, device)
    q = randn16((total, heads_q, head_dim), dtype, gd, device)
    k = randn16((total, heads_kv, head_dim), dtype, gd, device)
    v = randn16((total, heads_kv, head_dim), dtype, gd, device)
    cu_t = torch.tensor(cu, dtype=torch.int32, device=device)
    return q, k, v, cu_t, list(lengths)


def make_kvcache(seed, batch, seqlen_q, seqlen_k, heads_q, heads_kv, head_dim, dtype,
                 device="cpu", random_lengths=False, nan_tail=False):
    """q [B, Sq, Hq, D], caches [B, Sk, Hkv, D] and int32 cache_seqlens [B]."""
    g = _gen(seed, device)
    q = randn16((batch, seqlen_q, heads_q, head_dim), dtype, g, device)
    kc = randn16((batch, seqlen_k, heads_kv, head_dim), dtype, g, device)
    vc = randn16((batch, seqlen_k, heads_kv, head_dim), dtype, g, device)
    if random_lengths:
        gl = _gen(seed + 1, "cpu")
        lens = torch.randint(1, seqlen_k + 1, (batch,), generator=gl)
    else:
        lens = torch.full((batch,), seqlen_k, dtype=torch.int64)
    if nan_tail:
        for b in range(batch):
            n = int(lens[b])
            kc[b, n:] = float("nan")
            vc[b, n:] = float("nan")
    return q, kc, vc, lens.to(torch.int32).to(device)


def alibi_slopes(heads, batch=None, device="cpu"):
    """fp32 ALiBi slopes: the geometric sequence 2^(-8 (h + 1) / heads) over the query heads.

    With ``batch`` the result is [batch, heads], entry b scaled by (b + 1) / batch so that
    each batch row differs; otherwise [heads].  Input construction only.
    """
    base = torch.tensor([2.0 ** (-8.0 * (h + 1) / heads) for h in range(heads)], dtype=torch.float32)
    if batch is not None:
        base = torch.stack([base * (b + 1) / batch for b in range(batch)])
    return base.to(device)


def page_cache(kc, vc, lens, page, seed, spare_pages=3):
    """Scatter a contiguous cache [B, Sk, H, D] into a shuffled page pool.

    Returns (pool_k, pool_v [num_pages, page, H, D], table int32 [B, ceil(Sk/page)]):
    sequence b's i-th page lands in a random slot; spare slots and rows at or
    past lens[b] hold NaN (they must never be read).  Input construction only.
    """
    b_, sk, h, d = kc.shape
    per = -(-sk // page)
    n_pages = b_ * per + spare_pages
    g = torch.Generator(device="cpu").manual_seed(seed)
    slots = torch.randperm(n_pages, generator=g)
    pool_k = torch.full((n_pages, page, h, d), float("nan"), dtype=kc.dtype, device=kc.device)
    pool_v = torch.full_like(pool_k, float("nan"))
    table = torch.zeros((b_, per), dtype=torch.int32)
    lens_h = lens.cpu().tolist()
    for b in range(b_):
        for i in range(per):
            s = int(slots[b * per + i])
            table[b, i] = s
            lo, hi = i * page, min((i + 1) * page, sk, max(int(lens_h[b]), 0))
            if hi > lo:
                pool_k[s, :hi - lo] = kc[b, lo:hi]
                pool_v[s, :hi - lo] = vc[b, lo:hi]
    return pool_k, pool_v, table.to(kc.device)

