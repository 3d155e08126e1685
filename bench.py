#!/usr/bin/env python3
"""Benchmark of the q4g64 hot path on one MI355X.

One step is one decode FFN step at one activation row, with the workload's
sizes: qmv_w13_swiglu over w1 and w3 (8192 x 2048 each, bf16 x, float32
SwiGLU output), then qmv_rows over w2 (2048 x 8192) on that float32 output.
Weights rotate over a pool of packed copies larger than the 256 MB MALL plus
the L2s, so every step streams its 28 MB of weights from HBM, as a real
decode step streams the model's weights once per token.

The timed region replays a HIP graph of the K steps (host launch cost would
otherwise dominate a 10 us step), bracketed by torch.cuda.synchronize(). The
runtime cannot time events inside a graph, and an event between two decode
kernels costs about as much as the kernel, so each kernel's average duration
is taken over a graph of the same K launches of that kernel alone (same pool
rotation and buffers), bracketed by two HIP events on the stream it runs on.
The prompt GEMM is reported beside it (TFLOP/s against the bf16
matrix-core peak) on the 8192-row w1/w3 + SwiGLU window.

The float64 oracle is timed on the host on a bounded sample of the same
decode step (cpu_baseline).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
METRIC = "GB/s + rows/s for qmv decode; TFLOP/s for pgemm prefill (% of roofline)"


def qbytes(N, K, bits=4):
    """Algorithmic bytes of one packed matrix: bits/8 per code plus a bf16
    scale and bias (4 bytes) per 64 codes."""
    return N * K * (2 * bits + 1) // 16


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def to_dev(a, dt, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(dev)


def pack_dev(w, dev):
    import bit_weight_only_q4g64_amd as q4

    return q4.pack(to_dev(w.wq, np.int32, dev), to_dev(w.scales, np.int16, dev), to_dev(w.biases, np.int16, dev),
                   bits=getattr(w, "bits", 4))


def cpu_baseline(d, budget_s=12.0):
    """The float64 oracle on the same decode step, repeated while under budget."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count() or 1
    w1, w3, w2, x = d["w1"], d["w3"], d["w2"], d["x"]
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        a = oracle.matmul_rows(w1.wq, w1.scales, w1.biases, x)
        c = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, x)
        z = oracle.swiglu(a, c)
        oracle.matmul_rows(w2.wq, w2.scales, w2.biases, z)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 5:
            break
    step = float(np.median(times))
    nbytes = decode_step_bytes(d)
    out = {
        "value": nbytes / step / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(times)} full decode FFN steps (w1/w3 8192x2048 + SwiGLU, w2 2048x8192, 1 row) in numpy float64; "
        f"median {step * 1e3:.1f} ms per step",
    }
    # the same with the BLAS pool limited to one thread
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover - threadpoolctl missing
        return out
    times1 = []
    with threadpool_limits(limits=1):
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            a = oracle.matmul_rows(w1.wq, w1.scales, w1.biases, x)
            c = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, x)
            oracle.matmul_rows(w2.wq, w2.scales, w2.biases, oracle.swiglu(a, c))
            times1.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > budget_s or len(times1) >= 3:
                break
    step1 = float(np.median(times1))
    out["one_core"] = {"value": nbytes / step1 / 1e9, "unit": "GB/s", "cores": 1,
                       "sample": f"{len(times1)} steps, median {step1 * 1e3:.1f} ms per step"}
    return out


PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["bit_weight_only_q4g64_amd/csrc/common.h", "bit_weight_only_q4g64_amd/csrc/qmv.h",
                  "bit_weight_only_q4g64_amd/csrc/pgemm_narrow.h",
                  "bit_weight_only_q4g64_amd/csrc/pgemm.h", "bit_weight_only_q4g64_amd/csrc/api.hip"]


def _code_only(text):
    """C++ source without its comments and blank lines (string literals kept), so
    that editing a comment does not count as changing a kernel."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(line.rstrip() for line in "".join(out).splitlines() if line.strip())


def kernel_source_hash():
    """Hash of the kernel sources' code (comments and blank lines left out)."""
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_per_launch(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter on a plain copy
    of known size), or None when the summary is missing or was taken on
    different kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{kernel}.md")
    try:
        with open(path) as f:
            text = f.read()
        data = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if data.get("kernel_source_hash") != kernel_source_hash():
        return None
    return data.get("hbm_bytes_per_launch")


def copy_calibration(torch):
    """A plain device copy of a known size, for scaling the byte counters."""
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def batch_average_us(torch, launch, first, K):
    """Average device time per launch of K launches captured in one graph."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(K):
                launch(first + i)
    torch.cuda.synchronize()
    g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / K


def decode_step_bytes(d):
    w1, w2 = d["w1"], d["w2"]
    b13 = 2 * qbytes(w1.N, w1.K) + w1.K * 2 + w1.N * 4
    b2 = qbytes(w2.N, w2.K) + w2.K * 4 + w2.N * 4
    return b13 + b2


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--pool-mb", type=int, default=1200, help="size of the rotating weight pool (cold HBM reads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pgemm", action="store_true")
    ap.add_argument("--no-wide", action="store_true", help="skip the 6- and 8-bit measurements")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps directly instead of replaying a graph (for per-dispatch counters)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (the reference for scaling HBM byte counters)")
    ap.add_argument("--pgemm-only", action="store_true",
                    help="only the prompt GEMM measurement (for its per-dispatch counters); prints its JSON object")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (sharding is described in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.pgemm_only:
        import bit_weight_only_q4g64_amd as q4

        q4.lib()
        torch.cuda.set_device(0)
        print(json.dumps(bench_pgemm("cuda:0")))
        return

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    q4.lib()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log("generating the decode FFN workload")
    d = synthetic.config(1)
    w1, w3, w2 = d["w1"], d["w3"], d["w2"]
    copy_bytes = q4.packed_bytes(w1.N, w1.K) * 2 + q4.packed_bytes(w2.N, w2.K)
    ncopies = max(2, -(-args.pool_mb * (1 << 20) // copy_bytes))
    base = [pack_dev(w1, dev), pack_dev(w3, dev), pack_dev(w2, dev)]
    pool = [base] + [[t.clone() for t in base] for _ in range(ncopies - 1)]
    torch.cuda.synchronize()
    log(f"pool: {ncopies} copies of {copy_bytes / 1e6:.1f} MB = {ncopies * copy_bytes / 2**30:.2f} GiB")
    x = to_dev(d["x"], np.int16, dev).view(torch.bfloat16)
    z = torch.empty((1, w1.N), dtype=torch.float32, device=dev)
    y = torch.empty((1, w2.N), dtype=torch.float32, device=dev)

    def step(i, ev=None):
        p1, p3, p2 = pool[i % ncopies]
        if ev is not None:
            ev[0].record()
        q4.qmv_w13_swiglu(p1, p3, w1.N, w1.K, x, y=z)
        if ev is not None:
            ev[1].record()
        q4.qmv_rows(p2, w2.N, w2.K, z, y=y)
        if ev is not None:
            ev[2].record()

    K, W = args.steps, args.warmup
    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    # graph of K steps (each step on the next pool copy)
    g = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(K):
                    step(W + i)
        torch.cuda.synchronize()
        g.replay()  # untimed replay: first-launch costs
        torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]

    def run_timed():
        if g is not None:
            g.replay()
        else:
            for i in range(K):
                step(W + i, evs[i])

    log(f"timed region: {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_timed()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    if g is not None:
        # The runtime cannot time events inside a graph, and an event between
        # two kernels costs about as much as a decode kernel. Each kernel's
        # average duration is therefore taken over a graph of the same K
        # launches of that kernel alone (same pool rotation, same buffers),
        # bracketed by two events on the stream it runs on.
        t13 = np.array([batch_average_us(torch, lambda i: q4.qmv_w13_swiglu(pool[i % ncopies][0], pool[i % ncopies][1],
                                                                            w1.N, w1.K, x, y=z), W, K)])
        t2 = np.array([batch_average_us(torch, lambda i: q4.qmv_rows(pool[i % ncopies][2], w2.N, w2.K, z, y=y), W, K)])
        timing_src = "HIP events around a graph of the same K launches of each kernel alone, divided by K"
    else:
        t13 = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3  # us
        t2 = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e3
        timing_src = "HIP events around each kernel of the timed steps (launched directly)"

    b13 = 2 * qbytes(w1.N, w1.K) + w1.K * 2 + w1.N * 4
    b2 = qbytes(w2.N, w2.K) + w2.K * 4 + w2.N * 4
    step_bytes = b13 + b2
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    ach13 = b13 / (t13.mean() * 1e-6) / 1e9
    ach2 = b2 / (t2.mean() * 1e-6) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode FFN step: qmv_w13_swiglu over w1/w3 8192x2048 q4g64 + SwiGLU, then qmv_rows over w2 "
            "2048x8192 q4g64 on the float32 output; 1 bf16 activation row; seed 1",
            "rows": 1,
            "step_bytes": step_bytes,
            "weight_pool_gib": round(ncopies * copy_bytes / 2**30, 3),
            "kernel_source_hash": kernel_source_hash(),
            "timing": ("HIP graph of K steps" if g is not None else "K directly launched steps") + ", wall clock between synchronizes",
            "kernel_timing": timing_src,
        },
        "rows_per_s": round(1.0 / (ms_per_step * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "kernel": "qmv_w13_swiglu (qmv_kernel<0,2>)",
            "achieved": round(ach13, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(ach13 / HBM_PEAK_GBS, 4),
            "traffic": traffic_per_launch("qmv_w13_swiglu"),
            "algorithmic_bytes_per_launch": b13,
            "avg_launch_us": round(float(t13.mean()), 3),
        },
        "kernels": {
            "qmv_w13_swiglu": {"avg_us": round(float(t13.mean()), 3), "p10_us": round(float(np.percentile(t13, 10)), 3),
                               "p90_us": round(float(np.percentile(t13, 90)), 3), "GB/s": round(ach13, 1)},
            "qmv_rows_w2_f32x": {"avg_us": round(float(t2.mean()), 3), "p10_us": round(float(np.percentile(t2, 10)), 3),
                                 "p90_us": round(float(np.percentile(t2, 90)), 3), "GB/s": round(ach2, 1),
                                 "frac": round(ach2 / HBM_PEAK_GBS, 4), "traffic": traffic_per_launch("qmv_rows_w2"),
                                 "algorithmic_bytes_per_launch": b2},
        },
    }
    g_used = g is not None
    del g, pool
    torch.cuda.empty_cache()

    if not args.no_pgemm:
        result["pgemm"] = bench_pgemm(dev)
    if not args.no_wide:
        result["decode_rows"] = bench_rows(dev, K, W, args.pool_mb)
        r16 = result["decode_rows"]["R16"]
        result["rows_per_s_at_16_rows"] = max(r16["rows_per_s"], r16["planes_rows_per_s"], r16["tiled_rows_per_s"])
        result["qkv_rope"] = bench_qkv_rope(dev, K, W, args.pool_mb)
    if not args.no_wide:
        result["wide_codes"] = {str(b): bench_wide(dev, b, K, W, args.pool_mb, graph=g_used) for b in (6, 8, "fp8")}

    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host")
        result["cpu_baseline"] = cpu_baseline(d)
    print(json.dumps(result), flush=True)


def bench_wide(dev, bits, K, W, pool_mb, graph=True, reps=5):
    """The same decode FFN step and prompt window with MLX 6- or 8-bit codes,
    or block-FP8 weights (bits == "fp8"): same shapes, same cold weight pool,
    same timing method."""
    import torch

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    fp8 = bits == "fp8"
    log(f"{bits} weights: decode FFN step and prompt window")
    rng = np.random.default_rng(100 + (9 if fp8 else bits))
    if fp8:
        draw = lambda name, N, Kk: synthetic.draw_fp8_weight(rng, name, N, Kk)  # noqa: E731
        pack = lambda w: q4.pack_fp8b(to_dev(w.w8, np.uint8, dev), to_dev(w.scales, np.float32, dev))  # noqa: E731
        nbytes = q4.fp8b_packed_bytes
        w13_call = lambda p1, p3, x, z: q4.qmv_w13_swiglu_fp8b(p1, p3, 8192, 2048, x, y=z)  # noqa: E731
        rows_call = lambda p2, z, y: q4.qmv_rows_fp8b(p2, 2048, 8192, z, y=y)  # noqa: E731
        win_call = lambda p1, p3, xw, zw: q4.qmm_window_fp8b(p1, p3, 8192, 2048, xw, y=zw)  # noqa: E731
        algo = lambda N, Kk: N * Kk + 4 * N * Kk // 64  # noqa: E731  (one byte per weight + the 32-bit scale words)
    else:
        draw = lambda name, N, Kk: synthetic.draw_qweight(rng, name, N, Kk, bits=bits)  # noqa: E731
        pack = lambda w: pack_dev(w, dev)  # noqa: E731
        nbytes = lambda N, Kk: q4.packed_bytes(N, Kk, bits)  # noqa: E731
        w13_call = lambda p1, p3, x, z: q4.qmv_w13_swiglu(p1, p3, 8192, 2048, x, y=z, bits=bits)  # noqa: E731
        rows_call = lambda p2, z, y: q4.qmv_rows(p2, 2048, 8192, z, y=y, bits=bits)  # noqa: E731
        win_call = lambda p1, p3, xw, zw: q4.qmm_window(p1, p3, 8192, 2048, xw, y=zw, bits=bits)  # noqa: E731
        algo = lambda N, Kk: qbytes(N, Kk, bits)  # noqa: E731
    w1 = draw("w1", 8192, 2048)
    w3 = draw("w3", 8192, 2048)
    w2 = draw("w2", 2048, 8192)
    xb = synthetic.draw_bf16_rows(rng, 1, 2048)
    copy_bytes = nbytes(8192, 2048) * 2 + nbytes(2048, 8192)
    ncopies = max(2, -(-pool_mb * (1 << 20) // copy_bytes))
    base = [pack(w1), pack(w3), pack(w2)]
    pool = [base] + [[t.clone() for t in base] for _ in range(ncopies - 1)]
    x = to_dev(xb, np.int16, dev).view(torch.bfloat16)
    z = torch.empty((1, 8192), dtype=torch.float32, device=dev)
    y = torch.empty((1, 2048), dtype=torch.float32, device=dev)

    def step(i):
        p1, p3, p2 = pool[i % ncopies]
        w13_call(p1, p3, x, z)
        rows_call(p2, z, y)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(K):
                    step(W + i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        del g
    else:
        t0 = time.perf_counter()
        for i in range(K):
            step(W + i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / K
    t13 = batch_average_us(torch, lambda i: w13_call(pool[i % ncopies][0], pool[i % ncopies][1], x, z), W, K)
    t2 = batch_average_us(torch, lambda i: rows_call(pool[i % ncopies][2], z, y), W, K)
    b13 = 2 * algo(8192, 2048) + 2048 * 2 + 8192 * 4
    b2 = algo(2048, 8192) + 8192 * 4 + 2048 * 4
    del pool, base
    torch.cuda.empty_cache()

    # prompt window: w1/w3 + SwiGLU over 8192 rows, bf16 out
    xw = to_dev(synthetic.draw_bf16_rows(rng, 8192, 2048), np.int16, dev).view(torch.bfloat16)
    p1, p3 = pack(w1), pack(w3)
    zw = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        win_call(p1, p3, xw, zw)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    torch.cuda.synchronize()
    for e in evs:
        e[0].record()
        win_call(p1, p3, xw, zw)
        e[1].record()
    torch.cuda.synchronize()
    tw = np.array([e[0].elapsed_time(e[1]) for e in evs]).mean() * 1e-3
    tf = 2.0 * 8192 * (2 * 8192) * 2048 / tw / 1e12
    del p1, p3, zw, xw
    torch.cuda.empty_cache()
    return {
        "decode_step": {"ms_per_step": round(ms, 6), "GB/s": round((b13 + b2) / (ms * 1e-3) / 1e9, 2), "step_bytes": b13 + b2},
        "qmv_w13_swiglu": {"avg_us": round(t13, 3), "GB/s": round(b13 / (t13 * 1e-6) / 1e9, 1),
                           "frac": round(b13 / (t13 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "qmv_rows_w2_f32x": {"avg_us": round(t2, 3), "GB/s": round(b2 / (t2 * 1e-6) / 1e9, 1),
                             "frac": round(b2 / (t2 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "pgemm_swiglu_8192": {"avg_ms": round(tw * 1e3, 4), "TFLOP/s": round(tf, 2), "frac": round(tf / BF16_PEAK_TFLOPS, 4)},
    }


def bench_rows(dev, K, W, pool_mb):
    """The 4-bit decode FFN step with 2, 4, 8 and 16 activation rows sharing
    it (streams in one decode step): same shapes, cold weight pool and graph
    timing as the one-row step. rows/s = rows / step time."""
    import torch

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    log("decode FFN step at 2..16 rows")
    d = synthetic.config(1)
    w1, w3, w2 = d["w1"], d["w3"], d["w2"]
    copy_bytes = q4.packed_bytes(w1.N, w1.K) * 2 + q4.packed_bytes(w2.N, w2.K)
    ncopies = max(2, -(-pool_mb * (1 << 20) // copy_bytes))
    base = [pack_dev(w1, dev), pack_dev(w3, dev), pack_dev(w2, dev)]
    pool = [base] + [[t.clone() for t in base] for _ in range(ncopies - 1)]
    xs = to_dev(synthetic.draw_bf16_rows(np.random.default_rng(11), 16, w1.K), np.int16, dev).view(torch.bfloat16)
    z = torch.empty((16, w1.N), dtype=torch.float32, device=dev)
    y = torch.empty((16, w2.N), dtype=torch.float32, device=dev)
    z3s = {R: torch.empty((3, R, w1.N), dtype=torch.bfloat16, device=dev) for R in (1, 2, 4, 8, 16)}
    z3ts = {R: q4.TiledPlanes.empty(R, w1.N, dev) for R in (1, 2, 4, 8, 16)}
    out = {}
    for R in (1, 2, 4, 8, 16):
        z3 = z3s[R]

        def step(i):
            p1, p3, p2 = pool[i % ncopies]
            q4.qmv_w13_swiglu(p1, p3, w1.N, w1.K, xs[:R], y=z[:R])
            q4.qmv_rows(p2, w2.N, w2.K, z[:R], y=y[:R])

        def step3(i):
            p1, p3, p2 = pool[i % ncopies]
            q4.qmv_w13_swiglu(p1, p3, w1.N, w1.K, xs[:R], y=z3, planes=True)
            q4.qmv_rows(p2, w2.N, w2.K, z3, y=y[:R])

        z3t = z3ts[R]

        def step3t(i):
            p1, p3, p2 = pool[i % ncopies]
            q4.qmv_w13_swiglu(p1, p3, w1.N, w1.K, xs[:R], y=z3t, planes="tiled")
            q4.qmv_rows(p2, w2.N, w2.K, z3t, y=y[:R])

        us = batch_average_us(torch, step, W, K)
        us3 = batch_average_us(torch, step3, W, K)
        us3t = batch_average_us(torch, step3t, W, K)
        t13 = batch_average_us(torch, lambda i: q4.qmv_w13_swiglu(pool[i % ncopies][0], pool[i % ncopies][1], w1.N, w1.K, xs[:R],
                                                                  y=z[:R]), W, K)
        t2 = batch_average_us(torch, lambda i: q4.qmv_rows(pool[i % ncopies][2], w2.N, w2.K, z[:R], y=y[:R]), W, K)
        t2p = batch_average_us(torch, lambda i: q4.qmv_rows(pool[i % ncopies][2], w2.N, w2.K, z3, y=y[:R]), W, K)
        t2t = batch_average_us(torch, lambda i: q4.qmv_rows(pool[i % ncopies][2], w2.N, w2.K, z3t, y=y[:R]), W, K)
        b = 2 * qbytes(w1.N, w1.K) + qbytes(w2.N, w2.K) + R * (w1.K * 2 + w1.N * 4 + w2.K * 4 + w2.N * 4)
        out[f"R{R}"] = {"us_per_step": round(us, 3), "rows_per_s": round(R / (us * 1e-6), 1), "GB/s": round(b / (us * 1e-6) / 1e9, 1),
                        "qmv_w13_swiglu_us": round(t13, 3), "qmv_rows_w2_f32x_us": round(t2, 3),
                        "planes_us_per_step": round(us3, 3), "planes_rows_per_s": round(R / (us3 * 1e-6), 1),
                        "qmv_rows_w2_planes_us": round(t2p, 3),
                        "tiled_us_per_step": round(us3t, 3), "tiled_rows_per_s": round(R / (us3t * 1e-6), 1),
                        "qmv_rows_w2_tiled_us": round(t2t, 3)}
    del pool, base
    torch.cuda.empty_cache()
    out["workload"] = ("decode FFN step (w1/w3 8192x2048 + SwiGLU, w2 2048x8192, q4g64) with R bf16 rows, graph of K steps; "
                       "planes_*: the SwiGLU output handed to w2 as its three exact bf16 planes instead of float32 (same bits); "
                       "tiled_*: the same planes in the matvec's fragment order (Q4_BF16X3T, same bits)")
    return out


def bench_qkv_rope(dev, K, W, pool_mb):
    """The stacked q/k/v decode matvec (3072 x 2048, 4-bit) with partial RoPE
    and the KV store: fused in one launch against qmv_rows + rope_kv_store,
    at 1 and 16 rows, cold weights, graph-batch averages."""
    import torch

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    log("q/k/v matvec with RoPE and the KV store")
    d = synthetic.config(2)
    w = synthetic.concat_rows(d["wq"], d["wk"], d["wv"], name="qkv")
    base = pack_dev(w, dev)
    ncopies = max(2, -(-pool_mb * (1 << 20) // base.numel()))
    pool = [base] + [base.clone() for _ in range(ncopies - 1)]
    x = to_dev(d["x"], np.int16, dev).view(torch.bfloat16)
    ring = 4096
    pos = torch.arange(100, 116, dtype=torch.int32, device=dev)
    q = torch.empty((16, 2048), device=dev)
    kc = torch.empty((ring, 8, 64), device=dev, dtype=torch.bfloat16)
    vc = torch.empty((ring, 8, 64), device=dev, dtype=torch.bfloat16)
    y = torch.empty((16, w.N), device=dev)
    out = {}
    for R in (1, 16):
        fused = batch_average_us(torch, lambda i: q4.qmv_qkv_rope(pool[i % ncopies], w.K, x[:R], pos[:R], 32, 8, 64, 1e6, q[:R], kc, vc), W, K)

        def unfused(i):
            q4.qmv_rows(pool[i % ncopies], w.N, w.K, x[:R], y=y[:R])
            q4.rope_kv_store(y[:R], pos[:R], 32, 8, 64, 1e6, q[:R], kc, vc)

        two = batch_average_us(torch, unfused, W, K)
        mv = batch_average_us(torch, lambda i: q4.qmv_rows(pool[i % ncopies], w.N, w.K, x[:R], y=y[:R]), W, K)
        b = qbytes(w.N, w.K) + R * w.K * 2
        out[f"R{R}"] = {"fused_us": round(fused, 3), "qmv_rows_plus_epilogue_us": round(two, 3), "qmv_rows_alone_us": round(mv, 3),
                        "fused_GB/s": round(b / (fused * 1e-6) / 1e9, 1)}
    del pool, base
    torch.cuda.empty_cache()
    # gated attention: a gate projection of the q projection's shape stacked after v (the fourth matvec)
    wg = synthetic.draw_qweight(np.random.default_rng(951), "wg", 2048, 2048)
    w4 = synthetic.concat_rows(d["wq"], d["wk"], d["wv"], wg, name="qkvg")
    base = pack_dev(w4, dev)
    ncopies = max(2, -(-pool_mb * (1 << 20) // base.numel()))
    pool = [base] + [base.clone() for _ in range(ncopies - 1)]
    g = torch.empty((16, 2048), device=dev)
    y4 = torch.empty((16, w4.N), device=dev)
    for R in (1, 16):
        fused = batch_average_us(
            torch, lambda i: q4.qmv_qkv_rope(pool[i % ncopies], w4.K, x[:R], pos[:R], 32, 8, 64, 1e6, q[:R], kc, vc, gate_out=g[:R]), W, K)

        def unfused4(i):
            q4.qmv_rows(pool[i % ncopies], w4.N, w4.K, x[:R], y=y4[:R])
            q4.rope_kv_store(y4[:R], pos[:R], 32, 8, 64, 1e6, q[:R], kc, vc, gate_out=g[:R])

        two = batch_average_us(torch, unfused4, W, K)
        b = qbytes(w4.N, w4.K) + R * w4.K * 2
        out[f"gated_R{R}"] = {"fused_us": round(fused, 3), "qmv_rows_plus_epilogue_us": round(two, 3),
                              "fused_GB/s": round(b / (fused * 1e-6) / 1e9, 1)}
    del pool, base
    torch.cuda.empty_cache()
    out["workload"] = ("stacked q/k/v 3072x2048 q4g64 (32 q + 8 kv heads x 64), rot 64, theta 1e6, bf16 KV ring of 4096; "
                       "gated_*: q/k/v/gate 5120x2048 (32 gate heads after v)")
    return out


# HBM bytes the 8192-row w1/w3 + SwiGLU window must move at least: both
# packed weights once, the bf16 prompt once, the bf16 output once
PGEMM_BYTES = 2 * (8192 * 2048 * 9 // 16) + 8192 * 2048 * 2 + 8192 * 8192 * 2


def bench_pgemm(dev, reps=10):
    """w1/w3 + SwiGLU (bf16 out) over the 8192-row prompt as one window."""
    import torch

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    log("prompt GEMM: 8192 x (2 x 8192) x 2048 with SwiGLU")
    rng = np.random.default_rng(4)
    w1 = synthetic.draw_qweight(rng, "w1", 8192, 2048)
    w3 = synthetic.draw_qweight(rng, "w3", 8192, 2048)
    x = to_dev(synthetic.draw_bf16_rows(rng, 8192, 2048), np.int16, dev).view(torch.bfloat16)
    p1, p3 = pack_dev(w1, dev), pack_dev(w3, dev)
    z = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    for _ in range(2):
        q4.qmm_window(p1, p3, 8192, 2048, x, y=z)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    torch.cuda.synchronize()
    for e in evs:
        e[0].record()
        q4.qmm_window(p1, p3, 8192, 2048, x, y=z)
        e[1].record()
    torch.cuda.synchronize()
    t = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3  # s
    flops = 2.0 * 8192 * (2 * 8192) * 2048
    tf = flops / t.mean() / 1e12

    # the same prompt through the window driver in 128-row windows (64 short
    # windows, one launch each), checked bit for bit against the whole window
    log("prompt GEMM: the same 8192 rows as 64 windows of 128 rows (qmm_cut)")
    cut = [128] * 64
    zc = torch.empty_like(z)
    for _ in range(2):
        q4.qmm_cut(p1, p3, 8192, 2048, x, cut, y=zc)
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    torch.cuda.synchronize()
    for e in evc:
        e[0].record()
        q4.qmm_cut(p1, p3, 8192, 2048, x, cut, y=zc)
        e[1].record()
    torch.cuda.synchronize()
    tc = np.array([e[0].elapsed_time(e[1]) for e in evc]) * 1e-3
    same = bool(torch.equal(zc.view(torch.int16), z.view(torch.int16)))
    return {
        "workload": "qmm_window w1/w3 8192x2048 + SwiGLU, M=8192 prompt rows, bf16 out (seed 4 shapes)",
        "avg_ms": round(float(t.mean() * 1e3), 4),
        "TFLOP/s": round(tf, 2),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": traffic_per_launch("pgemm_swiglu_8192"),
                     "algorithmic_bytes_per_launch": PGEMM_BYTES},
        "windows_128": {
            "workload": "the same prompt through qmm_cut in 64 windows of 128 rows",
            "avg_ms": round(float(tc.mean() * 1e3), 4),
            "us_per_window": round(float(tc.mean() * 1e6 / 64), 2),
            "TFLOP/s": round(flops / tc.mean() / 1e12, 2),
            "bits_equal_whole_window": same,
        },
    }


if __name__ == "__main__":
    main()
