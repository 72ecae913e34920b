"""CPU checks of the host-side logic around the library: the FLOP count the benchmark divides by,
the seeded input generators and the paged-cache builder (no GPU, no library call)."""

import numpy as np
import pytest
import torch

import attn_workloads as W
import bench
import oracle


@pytest.mark.parametrize("sq,sk,causal,window", [
    (2048, 2048, True, (-1, -1)), (300, 500, True, (-1, -1)), (500, 300, True, (-1, -1)),
    (257, 257, False, (64, 0)), (128, 1000, False, (10, 20)), (64, 64, False, (0, 0)),
    (100, 100, False, (-1, -1)), (8192 // 16, 8192 // 16, True, (4096 // 16, 0)),
])
def test_visible_pairs_matches_mask(sq, sk, causal, window):
    """The benchmark's closed-form count of visible (query, key) pairs equals the oracle mask's."""
    mask = oracle.allowed_mask(sq, sk, np.arange(sq), causal, window[0], window[1])
    assert bench.visible_pairs(sq, sk, causal, window) == int(mask.sum())


def test_headline_flop_count():
    """cfg2: 2,098,176 visible pairs per head, 4 * D FLOP each, 64 heads."""
    c = W.WORKLOADS["cfg2_bf16_causal_2k"]
    pairs = bench.visible_pairs(c["seqlen_q"], c["seqlen_k"], c["causal"], c["window"])
    assert pairs == 2048 * 2049 // 2 == 2098176
    assert 4 * c["head_dim"] * pairs * c["batch"] * c["heads_q"] == 68753031168


def test_generators_are_seeded_and_16_bit():
    a = W.make_dense(5, 1, 33, 40, 4, 2, 64, "bf16")
    b = W.make_dense(5, 1, 33, 40, 4, 2, 64, "bf16")
    c = W.make_dense(6, 1, 33, 40, 4, 2, 64, "bf16")
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    assert a[0].shape == (1, 33, 4, 64) and a[1].shape == (1, 40, 2, 64)
    q, k, v, cu, lens = W.make_varlen(7, 5, 1, 1, 4, 2, 64, "fp16", lengths=[3, 0, 9, 1, 4])
    assert lens == [3, 0, 9, 1, 4] and cu.tolist() == [0, 3, 3, 12, 13, 17] and q.shape[0] == 17


def test_page_cache_round_trip():
    """Scattering a cache into shuffled pages and gathering it back (oracle side) is the identity on
    the valid rows; spare pages and rows past the valid length hold NaN."""
    q, kc, vc, lens = W.make_kvcache(8, 3, 1, 300, 2, 2, 64, "fp16", random_lengths=True)
    pk, pv, table = W.page_cache(kc, vc, lens, 64, 8, spare_pages=2)
    assert pk.shape[0] == 3 * 5 + 2 and table.shape == (3, 5)
    assert sorted(table.flatten().tolist()) == sorted(set(table.flatten().tolist()))
    for b in range(3):
        n = int(lens[b])
        got = oracle.gather_pages(pk.float().numpy(), table[b].numpy(), n)
        assert np.array_equal(got, kc[b, :n].float().numpy())
    used = set(table.flatten().tolist())
    spare = [s for s in range(pk.shape[0]) if s not in used]
    assert all(torch.isnan(pk[s]).all() for s in spare)


def test_alibi_slopes_geometric():
    s = W.alibi_slopes(8)
    assert s.dtype == torch.float32 and s.shape == (8,)
    assert torch.allclose(s, torch.tensor([2.0 ** (-(h + 1)) for h in range(8)]))
    sb = W.alibi_slopes(4, batch=2)
    assert sb.shape == (2, 4) and torch.allclose(sb[1], 2 * sb[0])
