#!/usr/bin/env python3
"""Benchmark of the exact tiled attention forward on one MI355X.

A step is one pass of the hot path over one batch of synthetic input resident
in HBM.  Default workload: fp16, B=4, Sq=Sk=4096, 32 query / 8 KV heads,
D=256, causal -- the configuration with the most algorithmic work that fits
one GPU.  Prints ONE JSON line with its throughput in TFLOP/s of algorithmic
work (4*D per visible query/key pair, i.e. causal pairs only), the roofline of
the dominant kernel against the published dense fp16 MFMA peak, the same
workload's fp64 CPU-oracle rate on a bounded sample, and every other
workload as a secondary measurement with its own fraction of roofline
(prefill TFLOP/s; decode HBM GB/s; the backward).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--warmup-floor-ms F] [--no-cpu-baseline] [--no-secondary]
                  [--mode copy|gemm|mfma]

Warm-up: W untimed steps, then more untimed steps until at least F ms
(default 200) of wall time has gone into them -- the GPU clock settles only
after ~20 ms of continuous work, so a fixed small W would time a ramping
clock.  ``--mode copy`` runs a plain device copy of known size instead; it is
the calibration kernel for the HBM byte counters (FETCH_SIZE / WRITE_SIZE).
``--mode gemm`` times the vendor's dense GEMM (torch.matmul, 16-bit, square
and wide shapes) with the same warm-up: the matrix-core rate this board
sustains once its clock has settled under full load, context for the
fraction of the published peak (not a bound the attention kernel is held to).
``--mode mfma`` does the same with nothing but back-to-back MFMAs (the debug
build's calibration kernel), on random and on zero operands.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s (4·B·H·Sq·Sk·D) & % MFMA peak; decode HBM GB/s"
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0}  # MI355X dense MFMA, published
PEAK_HBM_GBS = 8000.0                                  # MI355X HBM3E, published
HEADLINE = "cfg5b_fp16_d256_causal"
# Sources the forward tile kernel is compiled from (their hash keys the traffic records).
KERNEL_SRCS = [os.path.join(ROOT, "exact_tiled_attention_fa2_amd", "csrc", n)
               for n in ("attn_kernels.hip", "attn_device.h")]
# Per-workload HBM byte counts of the forward tile kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_{}.json")
WARMUP_FLOOR_MS = 200.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def visible_pairs(sq, sk, causal, window):
    """Number of visible (query, key) pairs of one head (bottom-right aligned band)."""
    import numpy as np

    i = np.arange(sq, dtype=np.int64)
    off = sk - sq
    hi = np.full(sq, sk - 1, dtype=np.int64)
    lo = np.zeros(sq, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, i + off)
    if window[1] >= 0:
        hi = np.minimum(hi, i + off + window[1])
    if window[0] >= 0:
        lo = np.maximum(lo, i + off - window[0])
    return int(np.clip(hi - lo + 1, 0, None).sum())


def kernel_sha():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload):
    """HBM bytes per launch from the committed counter summary of this workload, if the kernel
    sources are unchanged since the counters were taken (else None)."""
    try:
        with open(TRAFFIC_FILE.format(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_sha():
        return None
    return (t["fetch_kib_per_dispatch"] * t["fetch_scale"] + t["write_kib_per_dispatch"] * t["write_scale"]) * 1024.0


WARMUP_RUN = {}  # workload -> untimed steps actually run (W plus the floor's extra steps)


def time_region(fn, steps, warmup, torch, floor_ms=None, tag=None):
    """W untimed steps (then more until floor_ms of wall time has gone into warm-up), then K
    timed steps between synchronisations, with HIP events on the current stream (the stream the
    library launches on).  Returns ms per step."""
    floor_ms = WARMUP_FLOOR_MS if floor_ms is None else floor_ms
    t0 = time.perf_counter()
    ran = 0
    for _ in range(warmup):
        fn()
        ran += 1
    torch.cuda.synchronize()
    batch = 1
    while (time.perf_counter() - t0) * 1e3 < floor_ms:
        for _ in range(batch):
            fn()
        ran += batch
        torch.cuda.synchronize()
        batch = min(2 * batch, 64)
    if tag is not None:
        WARMUP_RUN[tag] = ran
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def cpu_baseline(cfg, budget_s=20.0):
    """The fp64 NumPy oracle, as is, on a bounded sample of the same workload: whole
    (batch, head) pairs in order until the budget is spent or the workload is done."""
    import torch

    import attn_workloads as W
    import oracle

    try:
        from threadpoolctl import threadpool_info
    except ImportError:  # pragma: no cover
        threadpool_info = None
    q, k, v = W.make_dense(cfg["seed"], cfg["batch"], cfg["seqlen_q"], cfg["seqlen_k"], cfg["heads_q"],
                           cfg["heads_kv"], cfg["head_dim"], cfg["dtype"], device="cpu",
                           k_ramp=cfg.get("k_ramp", False))
    g = cfg["heads_q"] // cfg["heads_kv"]
    sl = W.alibi_slopes(cfg["heads_q"]).to(torch.float64).numpy() if cfg.get("alibi") else None
    pairs = visible_pairs(cfg["seqlen_q"], cfg["seqlen_k"], cfg["causal"], cfg["window"])
    flops_head = 4.0 * cfg["head_dim"] * pairs
    total = cfg["batch"] * cfg["heads_q"]
    done, t0 = 0, time.perf_counter()
    while done < total:
        b, h = divmod(done, cfg["heads_q"])
        oracle.attention_ref(q[b:b + 1, :, h:h + 1].to(torch.float64).numpy(),
                             k[b:b + 1, :, h // g:h // g + 1].to(torch.float64).numpy(),
                             v[b:b + 1, :, h // g:h // g + 1].to(torch.float64).numpy(),
                             scale=cfg.get("scale"), causal=cfg["causal"], window=cfg["window"],
                             softcap=cfg["softcap"], alibi_slopes=None if sl is None else sl[h:h + 1])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = None
    if threadpool_info is not None:
        info = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        if info:
            threads = max(x.get("num_threads", 1) for x in info)
    return {"value": round(done * flops_head / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads if threads else os.cpu_count(), "kind": "oracle",
            "sample": f"{done} of {total} (batch, head) pairs of the workload"
                      f"{' (the whole workload)' if done == total else ''}, each a full "
                      f"{cfg['seqlen_q']}x{cfg['seqlen_k']} head, fp64 NumPy oracle, {dt:.1f} s",
            "host_cpus": os.cpu_count()}


def bench_dense(name, steps, warmup, torch, eng, W):
    c = W.WORKLOADS[name]
    q, k, v = W.make_dense(c["seed"], c["batch"], c["seqlen_q"], c["seqlen_k"], c["heads_q"],
                           c["heads_kv"], c["head_dim"], c["dtype"], k_ramp=c.get("k_ramp", False),
                           device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((c["batch"], c["heads_q"], c["seqlen_q"]), dtype=torch.float32, device="cuda")
    sl = W.alibi_slopes(c["heads_q"], device="cuda") if c.get("alibi") else None

    def step():
        eng.attn_fwd(q, k, v, causal=c["causal"], window=c["window"], softcap=c["softcap"],
                     softmax_scale=c.get("scale"), out=o, lse=lse, alibi_slopes=sl)

    ms = time_region(step, steps, warmup, torch, tag=name)
    pairs = visible_pairs(c["seqlen_q"], c["seqlen_k"], c["causal"], c["window"])
    flops = 4.0 * c["head_dim"] * pairs * c["batch"] * c["heads_q"]
    literal = 4.0 * c["batch"] * c["heads_q"] * c["seqlen_q"] * c["seqlen_k"] * c["head_dim"]
    config = {"workload": name, "batch": c["batch"], "seqlen_q": c["seqlen_q"], "seqlen_k": c["seqlen_k"],
              "heads_q": c["heads_q"], "heads_kv": c["heads_kv"], "head_dim": c["head_dim"],
              "causal": c["causal"], "window": list(c["window"]), "softcap": c["softcap"],
              "alibi": bool(c.get("alibi")), "flop_count": "4*D per visible (query, key) pair",
              "flops_per_step": flops, "literal_formula_flops_per_step": literal,
              "literal_formula_tflops": round(literal / (ms * 1e-3) / 1e12, 3)}
    return ms, flops, config, c


def bench_varlen(name, steps, warmup, torch, eng, W):
    c = W.WORKLOADS[name]
    q, k, v, cu, lens = W.make_varlen(c["seed"], c["n_seqs"], c["len_lo"], c["len_hi"], c["heads_q"],
                                      c["heads_kv"], c["head_dim"], c["dtype"], device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((c["heads_q"], q.shape[0]), dtype=torch.float32, device="cuda")
    mx = max(lens)

    def step():
        eng.attn_fwd_varlen(q, k, v, cu, cu, mx, mx, causal=c["causal"], window=c["window"],
                            softcap=c["softcap"], out=o, lse=lse)

    ms = time_region(step, steps, warmup, torch, tag=name)
    pairs = sum(visible_pairs(n, n, c["causal"], c["window"]) for n in lens)
    flops = 4.0 * c["head_dim"] * pairs * c["heads_q"]
    literal = sum(4.0 * c["heads_q"] * n * n * c["head_dim"] for n in lens)
    config = {"workload": name, "n_seqs": c["n_seqs"], "lengths": lens, "total_tokens": int(q.shape[0]),
              "heads_q": c["heads_q"], "heads_kv": c["heads_kv"], "head_dim": c["head_dim"],
              "causal": c["causal"], "flop_count": "4*D per visible (query, key) pair",
              "flops_per_step": flops, "literal_formula_flops_per_step": literal,
              "literal_formula_tflops": round(literal / (ms * 1e-3) / 1e12, 3)}
    return ms, flops, config, c


def bench_kvcache(name, steps, warmup, torch, eng, W):
    c = W.WORKLOADS[name]
    q, kc, vc, lens = W.make_kvcache(c["seed"], c["batch"], c["seqlen_q"], c["seqlen_k"], c["heads_q"],
                                     c["heads_kv"], c["head_dim"], c["dtype"], device="cuda")
    table = None
    if c.get("page"):  # the same cache scattered over a shuffled page pool
        kc, vc, table = W.page_cache(kc, vc, lens, c["page"], c["seed"])
        torch.cuda.empty_cache()
    o = torch.empty_like(q)
    lse = torch.empty((c["batch"], c["heads_q"], c["seqlen_q"]), dtype=torch.float32, device="cuda")
    ws = torch.empty(eng.attn_kvcache_workspace_bytes(c["batch"], c["seqlen_q"], c["heads_q"],
                                                      c["head_dim"], c["num_splits"]),
                     dtype=torch.uint8, device="cuda")
    sl = W.alibi_slopes(c["heads_q"], device="cuda") if c.get("alibi") else None

    def step():
        eng.attn_fwd_kvcache(q, kc, vc, cache_seqlens=lens, num_splits=c["num_splits"], out=o, lse=lse,
                             workspace=ws, block_table=table, alibi_slopes=sl)

    ms = time_region(step, steps, warmup, torch, tag=name)
    el = 2  # 16-bit
    bytes_alg = (2 * c["batch"] * c["seqlen_k"] * c["heads_kv"] * c["head_dim"] * el
                 + 2 * q.numel() * el + lse.numel() * 4)
    gbs = bytes_alg / (ms * 1e-3) / 1e9
    return {"workload": name, "ms_per_step": round(ms, 4), "value": round(gbs, 1), "unit": "GB/s",
            "bytes_per_step": bytes_alg, "num_splits": c["num_splits"],
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "peak": PEAK_HBM_GBS,
            "page_block_size": c.get("page"), "alibi": bool(c.get("alibi")),
            "note": "whole step (split kernel + combine); algorithmic bytes = K+V cache + Q + O + LSE"}


def bench_bwd(name, steps, warmup, torch, eng, W):
    """One attn_bwd call per step (the dot, dK/dV and dQ kernels); O and LSE come from one
    forward call before the timed region."""
    c = W.WORKLOADS[name]
    q, k, v = W.make_dense(c["seed"], c["batch"], c["seqlen_q"], c["seqlen_k"], c["heads_q"],
                           c["heads_kv"], c["head_dim"], c["dtype"], device="cuda")
    g = torch.Generator(device="cuda").manual_seed(c["seed"] + 7777)
    do = W.randn16(tuple(q.shape), c["dtype"], g, device="cuda")
    o, lse = eng.attn_fwd(q, k, v, causal=c["causal"], window=c["window"], softcap=c["softcap"])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(eng.attn_bwd_workspace_bytes(c["batch"], c["seqlen_q"], c["heads_q"]),
                     dtype=torch.uint8, device="cuda")

    def step():
        eng.attn_bwd(q, k, v, o, lse, do, causal=c["causal"], window=c["window"], softcap=c["softcap"],
                     dq=dq, dk=dk, dv=dv, workspace=ws)

    ms = time_region(step, steps, warmup, torch, tag=name)
    pairs = visible_pairs(c["seqlen_q"], c["seqlen_k"], c["causal"], c["window"])
    flops = 10.0 * c["head_dim"] * pairs * c["batch"] * c["heads_q"]
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[c["dtype"]]
    return {"workload": name, "ms_per_step": round(ms, 4), "value": round(tflops, 2), "unit": "TFLOP/s",
            "frac_of_mfma_peak": round(tflops / peak, 4), "peak": peak, "flops_per_step": flops,
            "note": "backward (dQ kernel, which also forms D, then dK/dV); algorithmic FLOPs = 10*D per visible pair "
                    "(five tile products); the kernels run seven (S and dP formed twice, no atomics)"}


# Forward latency table of the release page "v1.7 / flash_attn 2.9.2.post1", section 4.5
# (fp16, causal, one NVIDIA consumer GPU; batch and heads not stated): (S, D) -> ms per call.
PAGES_LATENCY_MS = {(1024, 64): 0.079, (1024, 128): 0.151, (4096, 64): 0.839, (4096, 128): 1.725,
                    (8192, 64): 3.162, (8192, 128): 6.504}


def run_pages_latency(steps, warmup, torch, eng, W):
    """The pages' latency shapes timed here (B = 2, H = 8 assumed: the page does not state them).
    Context only -- another machine, unknown batch and heads."""
    for (s, d), theirs in PAGES_LATENCY_MS.items():
        q, k, v = W.make_dense(2000 + s + d, 2, s, s, 8, 8, d, "fp16", device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((2, 8, s), dtype=torch.float32, device="cuda")

        def step():
            eng.attn_fwd(q, k, v, causal=True, out=o, lse=lse)

        ms = time_region(step, steps, warmup, torch)
        flops = 4.0 * d * visible_pairs(s, s, True, (-1, -1)) * 2 * 8
        print(json.dumps({"mode": "pages-latency", "seqlen": s, "head_dim": d, "batch": 2, "heads": 8,
                          "dtype": "fp16", "causal": True, "ms": round(ms, 4),
                          "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                          "pages_ms": theirs, "note": "pages: another GPU, batch/heads not stated"}),
              flush=True)
        del q, k, v, o, lse
        torch.cuda.empty_cache()


def run_copy(steps, warmup, torch):
    n = 1 << 30  # bytes per buffer
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    ms = time_region(lambda: b.copy_(a), steps, warmup, torch)
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "ms_per_copy": round(ms, 4),
                      "GBps_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def run_mfma(steps, warmup, torch):
    """The matrix-core rate this board sustains with nothing but back-to-back MFMAs (debug build's
    calibration kernel; no memory traffic, no other vector work), on random and on zero operands."""
    import ctypes
    from exact_tiled_attention_fa2_amd import debug
    h = debug.debug_lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 3 * cus, 20000  # 129 registers per lane: three waves per SIMD, one full round
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    for name, tdt, code in (("bf16", torch.bfloat16, 1), ("fp16", torch.float16, 0)):
        for fill in ("random", "zero"):
            g = torch.Generator(device="cuda")
            g.manual_seed(7)
            ops = (torch.randn(4096, device="cuda", generator=g) if fill == "random"
                   else torch.zeros(4096, device="cuda")).to(tdt)

            def step():
                rc = h.attn_debug_calib_mfma(code, ctypes.c_void_p(ops.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                             blocks, iters, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                if rc != 0:
                    raise RuntimeError(f"attn_debug_calib_mfma returned {rc}")

            ms = time_region(step, steps, warmup, torch)
            flops = float(blocks) * 4 * iters * 16 * 32768
            tf = flops / (ms * 1e-3) / 1e12
            print(json.dumps({"mode": "mfma", "dtype": name, "operands": fill, "workgroups": blocks, "iters": iters,
                              "ms": round(ms, 4), "tflops": round(tf, 1),
                              "frac_of_published_peak": round(tf / PEAK_MFMA_TFLOPS[name], 4),
                              "finite": bool(torch.isfinite(out).all().item()),
                              "note": "32x32x16 MFMAs only, four independent accumulators per wave"}),
                  flush=True)


def run_gemm(steps, warmup, torch):
    for dt in (torch.float16, torch.bfloat16):
        for m, n, k in ((8192, 8192, 8192), (16384, 16384, 8192), (8192, 8192, 16384)):
            a = torch.randn(m, k, device="cuda", dtype=dt)
            b = torch.randn(k, n, device="cuda", dtype=dt)
            c = torch.empty(m, n, device="cuda", dtype=dt)
            ms = time_region(lambda: torch.matmul(a, b, out=c), steps, warmup, torch)
            print(json.dumps({"mode": "gemm", "dtype": str(dt).replace("torch.", ""), "m": m, "n": n, "k": k,
                              "ms": round(ms, 4), "tflops": round(2.0 * m * n * k / (ms * 1e-3) / 1e12, 1),
                              "note": "torch.matmul (vendor GEMM), context only"}), flush=True)
            del a, b, c
            torch.cuda.empty_cache()


PREFILL_SECONDARY = ["cfg2_bf16_causal_2k", "cfg2r_bf16_causal_2k_kramp", "cfg3_bf16_varlen",
                     "cfg4_bf16_gqa_window_softcap"]


def prefill_entry(name, steps, warmup, torch, eng, W):
    """One prefill workload as a secondary record with its own fraction of the MFMA peak."""
    c = W.WORKLOADS[name]
    fn = bench_varlen if c["kind"] == "varlen" else bench_dense
    ms, flops, config, cfg = fn(name, steps, warmup, torch, eng, W)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[cfg["dtype"]]
    return {"workload": name, "ms_per_step": round(ms, 5), "value": round(tflops, 2), "unit": "TFLOP/s",
            "frac_of_mfma_peak": round(tflops / peak, 4), "peak": peak, "dtype": cfg["dtype"],
            "flops_per_step": flops, "literal_formula_tflops": config["literal_formula_tflops"],
            "traffic": load_traffic(name), "warmup_steps_run": WARMUP_RUN.get(name),
            "note": "one fwd_tile_kernel launch per step; algorithmic FLOPs = 4*D per visible pair"}


def main():
    global WARMUP_FLOOR_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--warmup-floor-ms", type=float, default=WARMUP_FLOOR_MS)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--mode", default="attn", choices=["attn", "copy", "gemm", "mfma", "pages-latency"])
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the forward shards over batch x KV-head groups with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import attn_workloads as W
    import exact_tiled_attention_fa2_amd as eng

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    WARMUP_FLOOR_MS = args.warmup_floor_ms
    eng.lib()
    if args.mode == "copy":
        run_copy(args.steps, args.warmup, torch)
        return
    if args.mode == "gemm":
        run_gemm(args.steps, args.warmup, torch)
        return
    if args.mode == "mfma":
        run_mfma(args.steps, args.warmup, torch)
        return
    if args.mode == "pages-latency":
        run_pages_latency(args.steps, args.warmup, torch, eng, W)
        return

    c = W.WORKLOADS[args.workload]
    log(f"workload {args.workload}: warmup {args.warmup} (floor {WARMUP_FLOOR_MS:g} ms), steps {args.steps}")
    if c["kind"] == "kvcache":
        sec = bench_kvcache(args.workload, args.steps, args.warmup, torch, eng, W)
        line = {"metric": METRIC, "value": sec["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": sec["ms_per_step"], "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": c["dtype"], "data": "synthetic",
                "config": {"workload": args.workload, **{k: c[k] for k in ("batch", "seqlen_q", "seqlen_k",
                                                                           "heads_q", "heads_kv", "head_dim",
                                                                           "num_splits")}},
                "roofline": {"bound": "hbm", "achieved": sec["value"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": sec["frac_of_hbm_peak"], "traffic": None},
                "warmup_steps_run": WARMUP_RUN.get(args.workload)}
        print(json.dumps(line), flush=True)
        return

    if c["kind"] == "bwd":
        sec = bench_bwd(args.workload, args.steps, args.warmup, torch, eng, W)
        line = {"metric": "attn bwd TFLOP/s (10*D per visible pair) & % MFMA peak", "value": sec["value"],
                "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                "ms_per_step": sec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": c["dtype"], "data": "synthetic",
                "config": {"workload": args.workload, **{k: c[k] for k in ("batch", "seqlen_q", "seqlen_k",
                                                                           "heads_q", "heads_kv", "head_dim",
                                                                           "causal")}},
                "roofline": {"bound": "mfma", "achieved": sec["value"], "peak": sec["peak"], "unit": "TFLOP/s",
                             "frac": sec["frac_of_mfma_peak"], "traffic": None,
                             "kernel": "bwd_dq (with D) + bwd_dkdv (one attn_bwd call per step)"},
                "warmup_steps_run": WARMUP_RUN.get(args.workload), "note": sec["note"]}
        print(json.dumps(line), flush=True)
        return

    if c["kind"] == "varlen":
        ms, flops, config, cfg = bench_varlen(args.workload, args.steps, args.warmup, torch, eng, W)
    else:
        ms, flops, config, cfg = bench_dense(args.workload, args.steps, args.warmup, torch, eng, W)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[cfg["dtype"]]
    log(f"{args.workload}: {ms:.4f} ms/step, {tflops:.1f} TFLOP/s")
    line = {"metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg["dtype"],
            "data": "synthetic", "config": config,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(tflops / peak, 4), "traffic": load_traffic(args.workload),
                         "kernel": "fwd_tile_kernel (one launch per step)"},
            "warmup_steps_run": WARMUP_RUN.get(args.workload)}
    if not args.no_secondary:
        line["secondary"] = []
        for name in PREFILL_SECONDARY:
            if name == args.workload:
                continue
            log(f"secondary: {name}")
            torch.cuda.empty_cache()
            line["secondary"].append(prefill_entry(name, args.steps, args.warmup, torch, eng, W))
        torch.cuda.empty_cache()
        log("secondary: cfg5a decode")
        dec = bench_kvcache("cfg5a_bf16_decode", args.steps, args.warmup, torch, eng, W)
        dec["warmup_steps_run"] = WARMUP_RUN.get("cfg5a_bf16_decode")
        line["secondary"].append(dec)
        torch.cuda.empty_cache()
        for name in ("bwd_cfg2_bf16_causal_2k", "bwd_cfg5b_fp16_d256_causal"):
            log(f"secondary: backward {name}")
            bwd = bench_bwd(name, args.steps, args.warmup, torch, eng, W)
            bwd["warmup_steps_run"] = WARMUP_RUN.get(name)
            line["secondary"].append(bwd)
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline and c["kind"] == "dense":
        log("cpu baseline (oracle on a bounded sample)")
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
