"""attn_fwd_kvcache_noalloc (split partials in the library's static per-GPU scratch) against
attn_fwd_kvcache (partials in a caller workspace): the same kernels and split count must give the
same bits.  Two calls in a row, the second smaller, so the second reads a scratch that still holds
the first call's partials; then a paged cache, and one split (no scratch at all)."""

import pytest
import torch

import attn_workloads as W
from gpu_common import gpu_required

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gpu_required()


def _eng():
    import exact_tiled_attention_fa2_amd as eng
    return eng


def _pair(q, kc, vc, lens, splits, **kw):
    eng = _eng()
    o_ref, l_ref = eng.attn_fwd_kvcache(q, kc, vc, cache_seqlens=lens, num_splits=splits, **kw)
    o = torch.full_like(q, float("nan"))
    lse = torch.full(l_ref.shape, float("nan"), dtype=torch.float32, device=q.device)
    eng.attn_fwd_kvcache_noalloc(q, kc, vc, o, lse, cache_seqlens=lens, num_splits=splits, **kw)
    torch.cuda.synchronize()
    return o_ref, l_ref, o, lse


def test_noalloc_matches_workspace_entry_two_calls():
    # first call: B=8, 4096-key caches, 32 / 8 heads, D=128, 16 splits (8 * 32 * 16 * 129 * 4 B of partials)
    print("[case] noalloc call 1: B=8 Sk=4096 32/8 heads D=128 bf16 16 splits", flush=True)
    q, kc, vc, lens = W.make_kvcache(71, 8, 1, 4096, 32, 8, 128, "bf16", device="cuda",
                                     random_lengths=True, nan_tail=True)
    o_ref, l_ref, o, lse = _pair(q, kc, vc, lens, 16, causal=True)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    # second call, smaller: B=3, 1000-key caches, 8 / 2 heads, D=64, fp16, 5 splits, 4 queries
    print("[case] noalloc call 2: B=3 Sq=4 Sk=1000 8/2 heads D=64 fp16 5 splits", flush=True)
    q2, kc2, vc2, lens2 = W.make_kvcache(72, 3, 4, 1000, 8, 2, 64, "fp16", device="cuda",
                                         random_lengths=True, nan_tail=True)
    o_ref2, l_ref2, o2, lse2 = _pair(q2, kc2, vc2, lens2, 5, causal=True)
    assert torch.equal(o2, o_ref2) and torch.equal(lse2, l_ref2)


def test_noalloc_paged_and_single_split():
    print("[case] noalloc paged: B=4 Sk=2048 16/4 heads D=128 bf16 7 splits, page 128", flush=True)
    q, kc, vc, lens = W.make_kvcache(73, 4, 1, 2048, 16, 4, 128, "bf16", device="cuda", random_lengths=True)
    pk, pv, table = W.page_cache(kc, vc, lens, 128, 73)
    o_ref, l_ref, o, lse = _pair(q, pk, pv, lens, 7, block_table=table)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    print("[case] noalloc single split", flush=True)
    o_ref, l_ref, o, lse = _pair(q, kc, vc, lens, 1)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_noalloc_rejects_oversize():
    """A split count whose partials exceed the scratch is refused before any launch."""
    eng = _eng()
    q, kc, vc, _ = W.make_kvcache(74, 32, 1, 8192, 32, 8, 128, "bf16", device="cuda")
    o = torch.zeros_like(q)
    with pytest.raises(RuntimeError, match="workspace"):
        eng.attn_fwd_kvcache_noalloc(q, kc, vc, o, num_splits=128)
    assert torch.all(o == 0)
