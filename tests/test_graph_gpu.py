"""The entry points captured in a HIP graph (torch.cuda.CUDAGraph) and replayed, and run
concurrently on two streams and from two host threads.

The library allocates nothing and enqueues no memset or copy: a call is its kernel launches on the
caller's stream, with the arguments fixed at the call.  So a captured call replays the same
kernels with the same launch arguments, and every replay must give the same bits as an eager call
on the same inputs.  Each graph is replayed three times; before each replay fresh inputs are
copied into the captured buffers, and after it the test makes the eager call and synchronises
(the program's own work between replays).  Workspaces and outputs that the binding allocates
during capture come from the graph's private memory pool and stay valid across replays.
"""

import pytest
import torch

import attn_workloads as W
from gpu_common import gpu_required

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gpu_required()


def _eng():
    import exact_tiled_attention_fa2_amd as eng
    return eng


def _bits(t):
    """The raw bits of a tensor (NaN-safe exact comparison)."""
    if t.element_size() == 2:
        return t.contiguous().view(torch.int16)
    if t.element_size() == 4:
        return t.contiguous().view(torch.int32)
    return t


def _check_replays(fn, buffers, fresh, what):
    """Capture fn() once, then for each replay copy fresh(i) into buffers, replay, and compare the
    graph's outputs bit for bit with an eager fn() on the same inputs."""
    print(f"[case] graph {what}", flush=True)
    fn()  # eager warm-up on the current stream: library loaded, per-device queries cached
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for dst, src in zip(buffers, fresh(i)):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        ref = fn()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(got, ref)):
            assert a.shape == b.shape
            assert torch.isfinite(a).any(), f"{what}: replay {i} output {j} holds no finite value"
            assert torch.equal(_bits(a), _bits(b)), f"{what}: replay {i} output {j} differs from the eager call"
    del g


@pytest.mark.parametrize("d,dtype,kw", [
    (128, "bf16", dict(causal=True)),
    (256, "fp16", dict(causal=True, softcap=30.0)),
    (64, "fp16", dict(window=(96, 32))),
])
def test_graph_fwd(d, dtype, kw):
    eng = _eng()
    q, k, v = W.make_dense(300 + d, 2, 700, 900, 8, 2, d, dtype, device="cuda")

    def fresh(i):
        return W.make_dense(310 + d + i, 2, 700, 900, 8, 2, d, dtype, device="cuda")

    _check_replays(lambda: eng.attn_fwd(q, k, v, **kw), [q, k, v], fresh, f"attn_fwd D={d} {dtype} {kw}")


def test_graph_fwd_varlen():
    eng = _eng()
    lens = [64, 700, 1, 333, 1024]
    q, k, v, cu, _ = W.make_varlen(320, len(lens), 0, 0, 8, 2, 128, "bf16", device="cuda", lengths=lens)
    mx = max(lens)

    def fresh(i):
        return W.make_varlen(321 + i, len(lens), 0, 0, 8, 2, 128, "bf16", device="cuda", lengths=lens)[:3]

    _check_replays(lambda: eng.attn_fwd_varlen(q, k, v, cu, cu, mx, mx, causal=True), [q, k, v], fresh,
                   "attn_fwd_varlen bf16 D=128 causal")


@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_kvcache(noalloc):
    eng = _eng()
    q, kc, vc, lens = W.make_kvcache(330, 4, 1, 4096, 32, 8, 128, "bf16", device="cuda",
                                     random_lengths=True, nan_tail=True)
    out = torch.empty_like(q)
    lse = torch.empty((4, 32, 1), dtype=torch.float32, device="cuda")

    def fresh(i):
        return W.make_kvcache(331 + i, 4, 1, 4096, 32, 8, 128, "bf16", device="cuda",
                              random_lengths=True, nan_tail=True)

    if noalloc:
        def fn():
            eng.attn_fwd_kvcache_noalloc(q, kc, vc, out, lse, cache_seqlens=lens, num_splits=16)
            return out, lse
    else:
        def fn():
            return eng.attn_fwd_kvcache(q, kc, vc, cache_seqlens=lens, num_splits=16)

    _check_replays(fn, [q, kc, vc, lens], fresh,
                   f"attn_fwd_kvcache{'_noalloc' if noalloc else ''} bf16 B=4 Sk=4096 16 splits")


def test_graph_bwd():
    eng = _eng()

    def make(seed):
        q, k, v = W.make_dense(seed, 2, 640, 640, 8, 2, 128, "bf16", device="cuda")
        o, lse = eng.attn_fwd(q, k, v, causal=True)
        do = W.randn16(o.shape, "bf16", W._gen(seed + 1, "cuda"), "cuda")
        return q, k, v, o, lse, do

    bufs = list(make(340))
    q, k, v, o, lse, do = bufs
    _check_replays(lambda: eng.attn_bwd(q, k, v, o, lse, do, causal=True), bufs,
                   lambda i: make(341 + i), "attn_bwd bf16 D=128 causal")


def test_two_streams_and_threads():
    """The library keeps no per-call state: calls interleaved on two streams, and issued from two
    host threads, give the same bits as the same calls one after another on one stream."""
    import threading
    eng = _eng()
    print("[case] two streams / two threads: forward D=128 and D=256, backward, decode", flush=True)
    qa, ka, va = W.make_dense(350, 2, 700, 700, 8, 2, 128, "bf16", device="cuda")
    qb, kb, vb = W.make_dense(351, 1, 500, 800, 8, 4, 256, "fp16", device="cuda")
    qc, kc, vc, lens = W.make_kvcache(352, 4, 1, 3000, 16, 4, 128, "bf16", device="cuda",
                                      random_lengths=True, nan_tail=True)
    do_a = W.randn16(tuple(qa.shape), "bf16", W._gen(353, "cuda"), "cuda")

    def job_a():
        o, l = eng.attn_fwd(qa, ka, va, causal=True)
        return [o, l, *eng.attn_bwd(qa, ka, va, o, l, do_a, causal=True)]

    def job_b():
        o, l = eng.attn_fwd(qb, kb, vb, causal=True, softcap=20.0)
        oc, lc = eng.attn_fwd_kvcache(qc, kc, vc, cache_seqlens=lens, num_splits=8)
        return [o, l, oc, lc]

    ref_a, ref_b = job_a(), job_b()
    torch.cuda.synchronize()

    def same(xs, ys):
        return all(torch.equal(_bits(x), _bits(y)) for x, y in zip(xs, ys))

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            outs.append(("a", job_a()))
        with torch.cuda.stream(s2):
            outs.append(("b", job_b()))
    torch.cuda.synchronize()
    for tag, xs in outs:
        assert same(xs, ref_a if tag == "a" else ref_b), f"stream run of job {tag} differs"

    results, errors = {}, []

    def worker(tag, fn):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                r = [fn() for _ in range(3)]
            s.synchronize()
            results[tag] = r
        except Exception as e:  # surfaced below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=("a", job_a)), threading.Thread(target=worker, args=("b", job_b))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for r in results["a"]:
        assert same(r, ref_a), "threaded run of job a differs"
    for r in results["b"]:
        assert same(r, ref_b), "threaded run of job b differs"
