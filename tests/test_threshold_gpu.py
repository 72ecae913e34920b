"""The rescale-threshold rule observed on the GPU, through the debug build's counters.

Page "v1.7 / flash_attn 2.9.2.post1", section 1.2: while a row's max rises by
at most the threshold (8 in log2 units for 16-bit inputs) the rescale of O
and the row sum is skipped and the max lags, so every P stays at or below
exp2(8) = 256 (fp16 holds 65504); page "FA2 2.9.0 Kernel Changes in v1.2",
section 3: the first KV step of a row never skips.  Outputs cannot show
which branch a row took (both are exact), so ``attn_fwd_stats`` of the debug
library counts, per query row, the steps that set the first max, skipped,
and rescaled, and records the largest P formed.  The counts are compared
with the tiled oracle (``oracle.tiled_ref(return_row_stats=True)``) run with
the kernel's own KV step, on the same inputs.  A decision within fp32
rounding of the threshold can go either way (the oracle is fp64), so a few
rows may differ; first-max and live-step counts are integer logic and must
match exactly.
"""

import numpy as np
import pytest
import torch

import attn_workloads as W
import oracle
from gpu_common import gpu_required, np64, run_jobs

pytestmark = pytest.mark.gpu

def p_bound(tau):
    """exp2(tau), with room for the rounding of the fp32 exponent."""
    return 2.0 ** tau * (1.0 + 2.0 ** -16)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gpu_required()


def _eng():
    import exact_tiled_attention_fa2_amd as eng
    return eng


CASES = [
    # (workload name, extra input options, threshold, sampled (batch, head) pairs)
    ("cfg2r_bf16_causal_2k_kramp", {}, 8.0, [(0, 0), (1, 5), (2, 9), (3, 15)]),
    ("cfg2_bf16_causal_2k", {}, 8.0, [(0, 3), (3, 12)]),
    ("cfg2r_bf16_causal_2k_kramp", {}, 0.0, [(0, 1), (2, 7)]),
    ("cfg2_bf16_causal_2k", {}, 0.0, [(1, 2)]),
    ("cfg5b_fp16_d256_causal", {}, 8.0, [(0, 0), (3, 31)]),
    ("cfg4_bf16_gqa_window_softcap", {"q_scale": 8.0}, 8.0, [(0, 0), (1, 17)]),
    # other thresholds the API accepts (0 to 15); at 15 in fp16 a lagging max lets P reach 2^15,
    # which fp16 still holds (65504), and the sampled heads are also checked against the oracle
    ("cfg2r_bf16_causal_2k_kramp", {}, 2.0, [(0, 0), (2, 9)]),
    ("cfg2r_bf16_causal_2k_kramp", {}, 4.0, [(1, 5)]),
    ("cfg2r_bf16_causal_2k_kramp", {"dtype": "fp16"}, 15.0, [(0, 0), (3, 15)]),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-tau{c[2]:g}{'-' + str(c[1]) if c[1] else ''}"
                                             for c in CASES])
def test_threshold_counters_match_oracle(case):
    from exact_tiled_attention_fa2_amd import debug
    name, extra, tau, pairs = case
    c = W.WORKLOADS[name]
    print(f"[case] threshold counters {name} tau={tau} {extra}", flush=True)
    extra = dict(extra)
    dtype = extra.pop("dtype", c["dtype"])
    q, k, v = W.make_dense(c["seed"], c["batch"], c["seqlen_q"], c["seqlen_k"], c["heads_q"], c["heads_kv"],
                           c["head_dim"], dtype, k_ramp=c.get("k_ramp", False), device="cuda", **extra)
    kw = dict(causal=c["causal"], window=c["window"], softcap=c["softcap"], rescale_threshold=tau)
    o_rel, l_rel = _eng().attn_fwd(q, k, v, **kw)
    o_dbg, l_dbg, st = debug.attn_fwd_stats(q, k, v, **kw)
    bk = debug.last_block_k()
    torch.cuda.synchronize()
    # the counters observe the release kernel's arithmetic without changing it
    assert torch.equal(o_rel, o_dbg) and torch.equal(l_rel, l_dbg)
    st = st.cpu().numpy()
    g = c["heads_q"] // c["heads_kv"]
    qn, kn, vn = np64(q), np64(k), np64(v)

    def ref(job):
        b, h = job
        *_, rs = oracle.tiled_ref(np.ascontiguousarray(qn[b:b + 1, :, h:h + 1]),
                                  np.ascontiguousarray(kn[b:b + 1, :, h // g:h // g + 1]),
                                  np.ascontiguousarray(vn[b:b + 1, :, h // g:h // g + 1]),
                                  causal=c["causal"], window=c["window"], softcap=c["softcap"], tau=tau,
                                  block_k=bk, return_row_stats=True)
        return rs

    tot = {"skips": 0, "rescales": 0, "ref_skips": 0, "ref_rescales": 0, "rows": 0, "differ": 0}
    pmax = 0.0
    for (b, h), rs in zip(pairs, run_jobs(ref, pairs)):
        kern = st[b, h]
        first, skips, resc = kern[:, 0].astype(np.int64), kern[:, 1].astype(np.int64), kern[:, 2].astype(np.int64)
        kp = kern[:, 3].copy().view(np.float32).astype(np.float64)
        assert np.array_equal(first, rs["first"][0, 0]), (b, h)
        assert np.array_equal(first + skips + resc, rs["first"][0, 0] + rs["skips"][0, 0] + rs["rescales"][0, 0]), \
            (b, h, "live steps")
        same = (skips == rs["skips"][0, 0]) & (resc == rs["rescales"][0, 0])
        tot["rows"] += same.size
        tot["differ"] += int((~same).sum())
        tot["skips"] += int(skips.sum())
        tot["rescales"] += int(resc.sum())
        tot["ref_skips"] += int(rs["skips"][0, 0].sum())
        tot["ref_rescales"] += int(rs["rescales"][0, 0].sum())
        assert np.all(np.isfinite(kp)) and np.all(kp <= p_bound(tau)), (b, h, float(kp.max()))
        # where the decisions agree, the largest P agrees to fp32 rounding
        rp = rs["max_p"][0, 0]
        assert np.all(np.abs(kp[same] - rp[same]) <= 1e-3 * np.maximum(rp[same], 1.0)), (b, h)
        pmax = max(pmax, float(kp.max()))
    print(f"[stats] {name} tau={tau} block_k={bk}: {tot} max P {pmax:.3f}", flush=True)
    assert tot["differ"] <= max(2, tot["rows"] // 1000), tot
    assert abs(tot["rescales"] - tot["ref_rescales"]) <= max(2, tot["ref_rescales"] // 200), tot
    assert tot["skips"] > 0
    if c.get("k_ramp") or tau == 0.0:
        assert tot["rescales"] > 0
    if tau >= 8.0 and c.get("k_ramp"):
        assert pmax > 16.0   # the lagging max lets P grow well above 1 on a rising max
    if tau == 15.0:
        def exact(job):
            b, h = job
            return oracle.attention_ref(np.ascontiguousarray(qn[b:b + 1, :, h:h + 1]),
                                        np.ascontiguousarray(kn[b:b + 1, :, h // g:h // g + 1]),
                                        np.ascontiguousarray(vn[b:b + 1, :, h // g:h // g + 1]),
                                        causal=c["causal"], window=c["window"], softcap=c["softcap"])
        on, ln = np64(o_rel), np64(l_rel)
        for (b, h), (ro, rl) in zip(pairs, run_jobs(exact, pairs)):
            r = oracle.compare(on[b:b + 1, :, h:h + 1], ro, ln[b:b + 1, h:h + 1], rl, dtype=dtype)
            print(f"[parity] tau=15 {dtype} ({b}, {h}): {r}", flush=True)
            assert r["pass"], (b, h, r)
