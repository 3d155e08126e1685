#!/usr/bin/env python3
"""Benchmark of the q4g64 hot path on one MI355X.

One step is one decode FFN step at one activation row, with the workload's
sizes: z = silu(W1 x) * (W3 x) over w1 and w3 (8192 x 2048 each, bf16 x),
then y = W2 z over w2 (2048 x 8192) on the float32 z. It runs as one launch
of qmv_ffn (the dataflow step, bit-identical to qmv_w13_swiglu followed by
qmv_rows). Weights rotate over a pool of packed copies of at least 1 GiB,
more than the 256 MB MALL plus the L2s, so every step streams its 28 MB of
weights from HBM, as a real decode step streams the model's weights once per
token.

The timed region replays a HIP graph of the K steps (host launch cost would
otherwise dominate a 12 us step), bracketed by torch.cuda.synchronize() for
the wall clock and by two HIP events on the graph's stream for the device
time of the step's kernel. Every other figure is the average over a graph of
at least as many launches as the pool has copies (so each timed graph reads
at least 1 GiB of weights), timed with two HIP events on the stream that
replays it.

Beside the headline, one line per workload: the single matvec (c0), the
attention projections at 1..16 rows (c2), the 1000-row prompt through every
cut (c3), the 8192-row layer with the 65536-row head (c4, as whole windows
and as 128-row windows), the decode step at 1..16 rows, the attention
epilogue and the 6-/8-bit and block-FP8 codes. The float64 oracle is timed
on the host on a bounded sample of the decode step (cpu_baseline), which also
reports the step's accuracy figures.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
METRIC = "GB/s + rows/s for qmv decode; TFLOP/s for pgemm prefill (% of roofline)"
POOL_BYTES = 1 << 30  # every rotating pool holds at least this many bytes


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


def rotating(base, min_bytes=POOL_BYTES, max_copies=None):
    """[base] plus clones of the list of device tensors `base`, totalling at
    least min_bytes (at least two copies)."""
    nbytes = sum(t.numel() * t.element_size() for t in base)
    n = max(2, -(-min_bytes // nbytes))
    if max_copies is not None:
        n = max(2, min(n, max_copies))
    return [base] + [[t.clone() for t in base] for _ in range(n - 1)]


def graph_us(torch, launch, n):
    """Average device time per launch of launch(0) .. launch(n - 1) captured
    in one graph: one untimed replay, then one replay between two HIP events
    on the stream that replays it."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                launch(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / n


def r3(v):
    return round(float(v), 3)


# ---------------------------------------------------------------- provenance


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "bit_weight_only_q4g64_amd", "csrc")
KERNEL_SOURCES = sorted(os.path.relpath(os.path.join(CSRC, f), ROOT) for f in os.listdir(CSRC) if f.endswith((".h", ".hip")))


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
    """Hash of the kernel sources' code (comments and blank lines left out) and
    of the compiler flags they are built with."""
    from bit_weight_only_q4g64_amd import build as _build

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    h.update(repr(_build.FLAGS).encode())
    return h.hexdigest()[:16]


def summary_json(name):
    """The machine-readable block of a committed profile summary, or None."""
    try:
        with open(os.path.join(PROFILES, name)) as f:
            text = f.read()
        return json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None


def traffic_per_launch(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter on a plain copy
    of known size), or None when the summary is missing or was taken on
    different kernel sources."""
    data = summary_json(f"traffic_{kernel}.md")
    if data is None or data.get("kernel_source_hash") != kernel_source_hash():
        return None
    return data.get("hbm_bytes_per_launch")


def _run(cmd):
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
        return r.stdout if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        return None


def provenance(torch, inputs):
    """Toolchain, device, clocks, host CPU and the SHA-256 of every input."""
    import bit_weight_only_q4g64_amd as q4

    p = {"kernel_source_hash": kernel_source_hash()}
    with open(q4.LIB_PATH, "rb") as f:
        p["library_sha256"] = hashlib.sha256(f.read()).hexdigest()
    out = _run(["hipcc", "--version"]) or _run(["/opt/rocm/bin/hipcc", "--version"])
    p["hipcc"] = [ln for ln in out.splitlines() if ln.strip()][:2] if out else None
    p["torch"] = torch.__version__
    p["hip_runtime"] = getattr(torch.version, "hip", None)
    props = torch.cuda.get_device_properties(0)
    p["device"] = {"name": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
                   "compute_units": props.multi_processor_count, "memory_gib": round(props.total_memory / 2**30, 1)}
    smi = _run(["rocm-smi", "--showclocks", "--json"])
    try:
        p["clocks"] = json.loads(smi) if smi else None
    except ValueError:
        p["clocks"] = smi.strip()[:2000] if smi else None
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    p["host_cpu"] = {"model": cpu, "cores_usable": len(os.sched_getaffinity(0))}
    p["inputs_sha256"] = inputs
    return p


def input_hashes(d):
    """SHA-256 of every canonical tensor of a workload dict."""
    import synthetic

    out = {}
    for k, v in d.items():
        if hasattr(v, "wq"):
            out[k] = {"wq": synthetic.sha256_of(v.wq), "scales": synthetic.sha256_of(v.scales),
                      "biases": synthetic.sha256_of(v.biases)}
        elif isinstance(v, np.ndarray):
            out[k] = synthetic.sha256_of(v)
    return out


# ------------------------------------------------------------ CPU baseline


def cpu_baseline(d, z_gpu, y_gpu, budget_s=12.0):
    """The float64 oracle on the same decode step, repeated while under
    budget, with the accuracy of the GPU's z and y against it."""
    import oracle
    from oracle.diagnostics import accuracy

    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count() or 1
    w1, w3, w2, x = d["w1"], d["w3"], d["w2"], d["x"]

    def step():
        a = oracle.matmul_rows(w1.wq, w1.scales, w1.biases, x)
        c = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, x)
        z = oracle.swiglu(a, c)
        return a, c, z, oracle.matmul_rows(w2.wq, w2.scales, w2.biases, z)

    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        a64, c64, z64, y64 = step()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 5:
            break
    med = float(np.median(times))
    nbytes = decode_step_bytes(d)
    out = {
        "value": nbytes / med / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(times)} full decode FFN steps (w1/w3 8192x2048 + SwiGLU, w2 2048x8192, 1 row) in numpy float64 "
        f"(dequantize, dgemm, silu); median {med * 1e3:.1f} ms per step",
    }
    # accuracy of the GPU step (reported, not gated): z against the float64
    # SwiGLU, y against the float64 chain
    Az = np.abs(oracle.silu(a64)) * oracle.error_weight(w3.wq, w3.scales, w3.biases, x) + \
        np.abs(c64) * oracle.error_weight(w1.wq, w1.scales, w1.biases, x)
    Ay = oracle.error_weight(w2.wq, w2.scales, w2.biases, np.abs(z64))
    out["accuracy"] = {"z": accuracy(z_gpu, z64, Az), "y": accuracy(y_gpu, y64, Ay),
                       "note": "z against the float64 SwiGLU; y against the float64 chain (float64 z into w2); "
                               "A: the error weight sum |w| |x| (for z, the first-order weight of the product)"}
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover - threadpoolctl missing
        return out
    times1 = []
    with threadpool_limits(limits=1):
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            step()
            times1.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > budget_s or len(times1) >= 3:
                break
    med1 = float(np.median(times1))
    out["one_core"] = {"value": nbytes / med1 / 1e9, "unit": "GB/s", "cores": 1,
                       "sample": f"{len(times1)} steps, median {med1 * 1e3:.1f} ms per step"}
    return out


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


def copy_bandwidth(torch):
    """Measured device-to-device copy rate (read + write bytes per second) of
    a 1 GiB buffer: context for the HBM peak."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) * 1e-3 / 5
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_each_way": n, "GB/s_read_plus_write": round(2 * n / s / 1e9, 1)}


# ----------------------------------------------------------- decode step


def decode_step_bytes(d, R=1):
    w1, w2 = d["w1"], d["w2"]
    b13 = 2 * qbytes(w1.N, w1.K) + R * (w1.K * 2 + w1.N * 4)
    b2 = qbytes(w2.N, w2.K) + R * (w2.K * 4 + w2.N * 4)
    return b13 + b2


def bench_step(d, dev, K, W, no_graph=False):
    """The headline: K decode FFN steps at one row, each one qmv_ffn launch on
    the next copy of a >= 1 GiB weight pool; and the same step as two calls."""
    import torch

    import bit_weight_only_q4g64_amd as q4

    w1, w3, w2 = d["w1"], d["w3"], d["w2"]
    pool = rotating([pack_dev(w1, dev), pack_dev(w3, dev), pack_dev(w2, dev)])
    nc = len(pool)
    torch.cuda.synchronize()
    log(f"decode step pool: {nc} copies = {nc * sum(t.numel() for t in pool[0]) / 2**30:.2f} GiB")
    x = to_dev(d["x"], np.int16, dev).view(torch.bfloat16)
    z = torch.empty((1, w1.N), dtype=torch.float32, device=dev)
    y = torch.empty((1, w2.N), dtype=torch.float32, device=dev)
    work = q4.ffn_workspace(w1.N, w2.N, 1, dev)

    def step(i):
        p1, p3, p2 = pool[i % nc]
        q4.qmv_ffn(p1, p3, p2, w1.N, w1.K, w2.N, x, work, z=z, y=y)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    g = None
    if not no_graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(K):
                    step(W + i)
        torch.cuda.synchronize()
        g.replay()  # untimed replay: first-launch costs
    # every copy once, in order, so the last copies touched are not the
    # timed region's first ones
    for i in range(nc):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timed region: {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    if g is not None:
        g.replay()
    else:
        for i in range(K):
            step(W + i)
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    step_kernel_us = e0.elapsed_time(e1) * 1e3 / K
    assert q4.ffn_error(work) == 0, "the decode step gave up waiting"
    z_out, y_out = z.cpu().numpy().astype(np.float64), y.cpu().numpy().astype(np.float64)
    # the same step as the two decode calls, and each of them alone
    n = max(K, nc)
    zz = torch.empty_like(z)

    def two(i):
        p1, p3, p2 = pool[i % nc]
        q4.qmv_w13_swiglu(p1, p3, w1.N, w1.K, x, y=zz)
        q4.qmv_rows(p2, w2.N, w2.K, zz, y=y)

    t_two = graph_us(torch, two, n)
    t13 = graph_us(torch, lambda i: q4.qmv_w13_swiglu(pool[i % nc][0], pool[i % nc][1], w1.N, w1.K, x, y=zz), n)
    t2 = graph_us(torch, lambda i: q4.qmv_rows(pool[i % nc][2], w2.N, w2.K, zz, y=y), n)
    ffn_alone = graph_us(torch, step, n)
    del g, pool
    torch.cuda.empty_cache()
    return {"ms_per_step": ms_per_step, "step_kernel_us": step_kernel_us, "ffn_graph_us": ffn_alone, "two_calls_us": t_two,
            "w13_us": t13, "w2_us": t2, "pool_copies": nc, "z": z_out, "y": y_out}


# --------------------------------------------------------------- workloads


def bench_c0(dev, K):
    """Workload 0: one 512 x 256 matvec at one row (latency-bound; reported)."""
    import torch

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    d = synthetic.config(0)
    w = d["w"]
    pool = rotating([pack_dev(w, dev)], min_bytes=300 << 20, max_copies=4096)
    nc = len(pool)
    x = to_dev(d["x"], np.int16, dev).view(torch.bfloat16)
    y = torch.empty((1, w.N), dtype=torch.float32, device=dev)
    us = graph_us(torch, lambda i: q4.qmv_rows(pool[i % nc][0], w.N, w.K, x, y=y), max(K, nc))
    b = qbytes(w.N, w.K) + w.K * 2 + w.N * 4
    del pool
    return {"workload": "qmv_rows 512x256 q4g64, 1 bf16 row (seed 0); pool of copies of 300 MB (more than the MALL)",
            "us": r3(us), "GB/s": round(b / (us * 1e-6) / 1e9, 1), "algorithmic_bytes": b,
            "frac": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "rows_per_s": round(1 / (us * 1e-6), 1)}


def bench_c2(dev, K):
    """Workload 2: the stacked q/k/v matvec (3072 x 2048) and o (2048 x 2048)
    on the same R bf16 rows, R = 1, 2, 4, 8, 16: the pair as one decode step,
    each matvec alone, rows/s and the fraction of the HBM peak."""
    import torch

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    d = synthetic.config(2)
    qkv = synthetic.concat_rows(d["wq"], d["wk"], d["wv"], name="qkv")
    wo = d["wo"]
    pool = rotating([pack_dev(qkv, dev), pack_dev(wo, dev)])
    nc = len(pool)
    xs = to_dev(d["x"], np.int16, dev).view(torch.bfloat16)
    yq = torch.empty((16, qkv.N), dtype=torch.float32, device=dev)
    yo = torch.empty((16, wo.N), dtype=torch.float32, device=dev)
    n = max(K, nc)
    out = {"workload": "qkv 3072x2048 (32 q + 8 kv heads x 64) then o 2048x2048 on the same R bf16 rows, q4g64, seed 2; "
                       f"pool {nc} copies of both ({nc * (qbytes(3072, 2048) + qbytes(2048, 2048)) / 2**30:.2f} GiB)"}
    for R in (1, 2, 4, 8, 16):
        x = xs[:R]

        def pair(i):
            q4.qmv_rows(pool[i % nc][0], qkv.N, qkv.K, x, y=yq[:R])
            q4.qmv_rows(pool[i % nc][1], wo.N, wo.K, x, y=yo[:R])

        t = graph_us(torch, pair, n)
        tq = graph_us(torch, lambda i: q4.qmv_rows(pool[i % nc][0], qkv.N, qkv.K, x, y=yq[:R]), n)
        to = graph_us(torch, lambda i: q4.qmv_rows(pool[i % nc][1], wo.N, wo.K, x, y=yo[:R]), n)
        bq = qbytes(qkv.N, qkv.K) + R * (qkv.K * 2 + qkv.N * 4)
        bo = qbytes(wo.N, wo.K) + R * (wo.K * 2 + wo.N * 4)
        out[f"R{R}"] = {"pair_us": r3(t), "rows_per_s": round(R / (t * 1e-6), 1), "GB/s": round((bq + bo) / (t * 1e-6) / 1e9, 1),
                        "frac": round((bq + bo) / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "qkv_us": r3(tq), "qkv_frac": round(bq / (tq * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "o_us": r3(to), "o_frac": round(bo / (to * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del pool
    torch.cuda.empty_cache()
    return out


def bench_c3(dev, K):
    """Workload 3: the 1000-row prompt through w1/w3 with the SwiGLU epilogue
    (float32 out) as one window and through the cuts 64, 128, 256 and
    {17, 300, 683}; TFLOP/s per cut and the bits of every cut against the
    whole window."""
    import torch

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    d = synthetic.config(3)
    w1, w3 = d["w1"], d["w3"]
    M = d["x"].shape[0]
    pool = rotating([pack_dev(w1, dev), pack_dev(w3, dev), to_dev(d["x"], np.int16, dev).view(torch.bfloat16)])
    nc = len(pool)
    y = torch.empty((M, w1.N), dtype=torch.float32, device=dev)
    ref = q4.qmm_window(pool[0][0], pool[0][1], w1.N, w1.K, pool[0][2])
    torch.cuda.synchronize()
    flops = 2.0 * M * (2 * w1.N) * w1.K
    out = {"workload": f"qmm_window/qmm_cut w1/w3 8192x2048 + SwiGLU, {M} bf16 rows, float32 out, seed 3; "
                       f"pool {nc} copies of the weights and prompt"}
    cuts = {"whole": [M], **d["cuts"]}
    for name, cut in cuts.items():
        us = graph_us(torch, lambda i: q4.qmm_cut(pool[i % nc][0], pool[i % nc][1], w1.N, w1.K, pool[i % nc][2], cut, y=y), nc)
        tf = flops / (us * 1e-6) / 1e12
        out[name] = {"windows": len(cut), "us": r3(us), "TFLOP/s": round(tf, 2), "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                     "bits_equal_whole_window": bool(torch.equal(y.view(torch.int32), ref.view(torch.int32)))}
    del pool
    torch.cuda.empty_cache()
    return out


C4_FLOPS = {"qkv": 2.0 * 8192 * 3072 * 2048, "o": 2.0 * 8192 * 2048 * 2048, "w1w3_swiglu": 2.0 * 8192 * 16384 * 2048,
            "w2": 2.0 * 8192 * 2048 * 8192, "head": 2.0 * 128 * 65536 * 2048}


def bench_c4(dev, reps=4):
    """Workload 4: one decoder layer's projections over an 8192-row prompt
    (qkv, o, w1/w3 + SwiGLU with bf16 out, w2 on that output) and the 65536 x
    2048 head on the last 128 rows; once as whole windows and once in 128-row
    windows (qmm_cut). Two copies of the weights and prompt alternate, so a
    copy is read again only after the other's whole layer (over 0.5 GB of
    traffic) has passed."""
    import torch

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    log("c4: generating the 8192-row layer")
    d = synthetic.config(4)
    hashes = input_hashes(d)
    qkv = synthetic.concat_rows(d["wq"], d["wk"], d["wv"], name="qkv")
    ws = {"qkv": qkv, "o": d["wo"], "w1": d["w1"], "w3": d["w3"], "w2": d["w2"], "head": d["head"]}
    copies = []
    for c in range(2):
        pk = {k: pack_dev(w, dev) for k, w in ws.items()}
        pk["x"] = to_dev(d["x"], np.int16, dev).view(torch.bfloat16)
        copies.append(pk)
    M = d["x"].shape[0]
    yq = torch.empty((M, qkv.N), dtype=torch.float32, device=dev)
    yo = torch.empty((M, 2048), dtype=torch.float32, device=dev)
    z = torch.empty((M, 8192), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty((M, 2048), dtype=torch.float32, device=dev)
    yh = torch.empty((128, 65536), dtype=torch.float32, device=dev)
    cut = [128] * (M // 128)

    def ops(pk, windows):
        cq = cut if windows else [M]
        return [
            ("qkv", lambda: q4.qmm_cut(pk["qkv"], None, qkv.N, 2048, pk["x"], cq, y=yq)),
            ("o", lambda: q4.qmm_cut(pk["o"], None, 2048, 2048, pk["x"], cq, y=yo)),
            ("w1w3_swiglu", lambda: q4.qmm_cut(pk["w1"], pk["w3"], 8192, 2048, pk["x"], cq, y=z, out_dtype=torch.bfloat16)),
            ("w2", lambda: q4.qmm_cut(pk["w2"], None, 2048, 8192, z, cq, y=y2)),
            ("head", lambda: q4.qmm_window(pk["head"], None, 65536, 2048, pk["x"][-128:], y=yh)),
        ]

    out = {"workload": "8192-row layer: qkv 3072x2048, o 2048x2048, w1/w3 8192x2048 + SwiGLU (bf16 out), w2 2048x8192 on it, "
                       "then the 65536x2048 head on the last 128 rows; q4g64, seed 4; two alternating copies",
           "layer_gflop": round(sum(C4_FLOPS.values()) / 1e9, 1), "inputs_sha256": hashes}
    whole_bits = None
    for windows in (False, True):
        times = {k: [] for k in C4_FLOPS}
        for rep in range(reps + 1):
            pk = copies[rep % 2]
            evs = []
            for name, fn in ops(pk, windows):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                evs.append((name, e0, e1))
            torch.cuda.synchronize()
            if rep > 0:  # the first pass is a warm-up
                for name, e0, e1 in evs:
                    times[name].append(e0.elapsed_time(e1) * 1e-3)
        bits = [t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).clone() for t in (yq, yo, z, y2, yh)]
        if whole_bits is None:
            whole_bits = bits
        key = "windows_128" if windows else "whole"
        res = {}
        total = 0.0
        for name, ts in times.items():
            t = float(np.median(ts))
            total += t
            tf = C4_FLOPS[name] / t / 1e12
            res[name] = {"us": round(t * 1e6, 2), "TFLOP/s": round(tf, 2), "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
        tf = sum(C4_FLOPS.values()) / total / 1e12
        res["layer"] = {"us": round(total * 1e6, 2), "TFLOP/s": round(tf, 2), "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
        if windows:
            res["bits_equal_whole"] = all(bool(torch.equal(a, b)) for a, b in zip(bits, whole_bits))
        out[key] = res
    del copies
    torch.cuda.empty_cache()
    return out


def bench_rows(dev, K):
    """The decode FFN step with R = 1, 2, 4, 8, 16 rows sharing it: qmv_ffn
    (one launch up to 2 rows, the two calls with the fragment-ordered handoff
    beyond), and the two calls with the float32 or fragment-ordered
    (Q4_BF16X3T) handoff."""
    import torch

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    d = synthetic.config(1)
    w1, w3, w2 = d["w1"], d["w3"], d["w2"]
    pool = rotating([pack_dev(w1, dev), pack_dev(w3, dev), pack_dev(w2, dev)])
    nc = len(pool)
    n = max(K, nc)
    xs = to_dev(synthetic.draw_bf16_rows(np.random.default_rng(11), 16, w1.K), np.int16, dev).view(torch.bfloat16)
    z = torch.empty((16, w1.N), dtype=torch.float32, device=dev)
    y = torch.empty((16, w2.N), dtype=torch.float32, device=dev)
    work = q4.ffn_workspace(w1.N, w2.N, 16, dev)
    out = {"workload": "decode FFN step (w1/w3 8192x2048 + SwiGLU, w2 2048x8192, q4g64) with R bf16 rows; "
                       "graph averages over a >= 1 GiB pool"}
    for R in (1, 2, 4, 8, 16):
        x = xs[:R]
        t_ffn = graph_us(torch, lambda i: q4.qmv_ffn(pool[i % nc][0], pool[i % nc][1], pool[i % nc][2], w1.N, w1.K, w2.N, x, work,
                                                   z=z[:R], y=y[:R]), n)

        def two(i):
            q4.qmv_w13_swiglu(pool[i % nc][0], pool[i % nc][1], w1.N, w1.K, x, y=z[:R])
            q4.qmv_rows(pool[i % nc][2], w2.N, w2.K, z[:R], y=y[:R])

        zt = q4.TiledPlanes.empty(R, w1.N, dev)

        def two_tiled(i):
            q4.qmv_w13_swiglu(pool[i % nc][0], pool[i % nc][1], w1.N, w1.K, x, y=zt, planes="tiled")
            q4.qmv_rows(pool[i % nc][2], w2.N, w2.K, zt, y=y[:R])

        t_two = graph_us(torch, two, n)
        t_tiled = graph_us(torch, two_tiled, n)
        b = decode_step_bytes(d, R)
        best = min(t_ffn, t_two, t_tiled)
        out[f"R{R}"] = {"qmv_ffn_us": r3(t_ffn), "two_calls_us": r3(t_two), "two_calls_tiled_us": r3(t_tiled),
                        "best_rows_per_s": round(R / (best * 1e-6), 1), "best_GB/s": round(b / (best * 1e-6) / 1e9, 1)}
    assert q4.ffn_error(work) == 0
    del pool
    torch.cuda.empty_cache()
    return out


def bench_qkv_rope(dev, K):
    """The stacked q/k/v decode matvec (3072 x 2048, 4-bit) with partial RoPE
    and the KV store: fused in one launch against qmv_rows + rope_kv_store,
    at 1 and 16 rows; and with 32 gate heads stacked after v."""
    import torch

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    d = synthetic.config(2)
    wg = synthetic.draw_qweight(np.random.default_rng(951), "wg", 2048, 2048)
    x = to_dev(d["x"], np.int16, dev).view(torch.bfloat16)
    ring = 4096
    pos = torch.arange(100, 116, dtype=torch.int32, device=dev)
    q = torch.empty((16, 2048), device=dev)
    kc = torch.empty((ring, 8, 64), device=dev, dtype=torch.bfloat16)
    vc = torch.empty((ring, 8, 64), device=dev, dtype=torch.bfloat16)
    g = torch.empty((16, 2048), device=dev)
    out = {"workload": "stacked q/k/v 3072x2048 q4g64 (32 q + 8 kv heads x 64), rot 64, theta 1e6, bf16 KV ring of 4096; "
                       "gated_*: q/k/v/gate 5120x2048 (32 gate heads after v)"}
    for tag, w in (("", synthetic.concat_rows(d["wq"], d["wk"], d["wv"], name="qkv")),
                   ("gated_", synthetic.concat_rows(d["wq"], d["wk"], d["wv"], wg, name="qkvg"))):
        pool = rotating([pack_dev(w, dev)])
        nc = len(pool)
        n = max(K, nc)
        yy = torch.empty((16, w.N), device=dev)
        gate = g if tag else None
        for R in (1, 16):
            fused = graph_us(torch, lambda i: q4.qmv_qkv_rope(pool[i % nc][0], w.K, x[:R], pos[:R], 32, 8, 64, 1e6, q[:R], kc, vc,
                                                              gate_out=None if gate is None else gate[:R]), n)

            def unfused(i):
                q4.qmv_rows(pool[i % nc][0], w.N, w.K, x[:R], y=yy[:R])
                q4.rope_kv_store(yy[:R], pos[:R], 32, 8, 64, 1e6, q[:R], kc, vc, gate_out=None if gate is None else gate[:R])

            two = graph_us(torch, unfused, n)
            mv = graph_us(torch, lambda i: q4.qmv_rows(pool[i % nc][0], w.N, w.K, x[:R], y=yy[:R]), n)
            out[f"{tag}R{R}"] = {"fused_us": r3(fused), "qmv_rows_plus_epilogue_us": r3(two), "qmv_rows_alone_us": r3(mv)}
        del pool
        torch.cuda.empty_cache()
    return out


def bench_wide(dev, bits, K):
    """The decode FFN step (two calls), the 8192-row w1/w3 window and 128-row
    windows of w1/w3 and w2 with MLX 6- or 8-bit codes or block-FP8 weights
    (bits == "fp8"): same shapes, pool and timing as the 4-bit figures."""
    import torch

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    fp8 = bits == "fp8"
    rng = np.random.default_rng(100 + (9 if fp8 else bits))
    if fp8:
        draw = lambda name, N, Kk: synthetic.draw_fp8_weight(rng, name, N, Kk)  # noqa: E731
        pack = lambda w: q4.pack_fp8b(to_dev(w.w8, np.uint8, dev), to_dev(w.scales, np.float32, dev))  # noqa: E731
        w13_call = lambda p1, p3, x, z: q4.qmv_w13_swiglu_fp8b(p1, p3, 8192, 2048, x, y=z)  # noqa: E731
        rows_call = lambda p2, z, y: q4.qmv_rows_fp8b(p2, 2048, 8192, z, y=y)  # noqa: E731
        win_call = lambda p1, p3, xw, zw: q4.qmm_window_fp8b(p1, p3, 8192, 2048, xw, y=zw)  # noqa: E731
        w2win_call = lambda p2, xw, yw: q4.qmm_window_fp8b(p2, None, 2048, 8192, xw, y=yw)  # noqa: E731
        algo = lambda N, Kk: N * Kk + 4 * N * Kk // 64  # noqa: E731  (one byte per weight + the 32-bit scale words)
    else:
        draw = lambda name, N, Kk: synthetic.draw_qweight(rng, name, N, Kk, bits=bits)  # noqa: E731
        pack = lambda w: pack_dev(w, dev)  # noqa: E731
        w13_call = lambda p1, p3, x, z: q4.qmv_w13_swiglu(p1, p3, 8192, 2048, x, y=z, bits=bits)  # noqa: E731
        rows_call = lambda p2, z, y: q4.qmv_rows(p2, 2048, 8192, z, y=y, bits=bits)  # noqa: E731
        win_call = lambda p1, p3, xw, zw: q4.qmm_window(p1, p3, 8192, 2048, xw, y=zw, bits=bits)  # noqa: E731
        w2win_call = lambda p2, xw, yw: q4.qmm_window(p2, None, 2048, 8192, xw, y=yw, bits=bits)  # noqa: E731
        algo = lambda N, Kk: qbytes(N, Kk, bits)  # noqa: E731
    w1, w3, w2 = draw("w1", 8192, 2048), draw("w3", 8192, 2048), draw("w2", 2048, 8192)
    pool = rotating([pack(w1), pack(w3), pack(w2)])
    nc = len(pool)
    n = max(K, nc)
    x = to_dev(synthetic.draw_bf16_rows(rng, 1, 2048), np.int16, dev).view(torch.bfloat16)
    z = torch.empty((1, 8192), dtype=torch.float32, device=dev)
    y = torch.empty((1, 2048), dtype=torch.float32, device=dev)

    def step(i):
        w13_call(pool[i % nc][0], pool[i % nc][1], x, z)
        rows_call(pool[i % nc][2], z, y)

    t_step = graph_us(torch, step, n)
    t13 = graph_us(torch, lambda i: w13_call(pool[i % nc][0], pool[i % nc][1], x, z), n)
    t2 = graph_us(torch, lambda i: rows_call(pool[i % nc][2], z, y), n)
    b13 = 2 * algo(8192, 2048) + 2048 * 2 + 8192 * 4
    b2 = algo(2048, 8192) + 8192 * 4 + 2048 * 4
    # 128-row windows (the short-window kernels) on the rotating pool
    x128 = to_dev(synthetic.draw_bf16_rows(rng, 128, 2048), np.int16, dev).view(torch.bfloat16)
    x128w2 = to_dev(synthetic.draw_bf16_rows(rng, 128, 8192), np.int16, dev).view(torch.bfloat16)
    z128 = torch.empty((128, 8192), dtype=torch.bfloat16, device=dev)
    y128 = torch.empty((128, 2048), dtype=torch.float32, device=dev)
    t128_13 = graph_us(torch, lambda i: win_call(pool[i % nc][0], pool[i % nc][1], x128, z128), n)
    t128_2 = graph_us(torch, lambda i: w2win_call(pool[i % nc][2], x128w2, y128), n)
    f128_13 = 2.0 * 128 * (2 * 8192) * 2048 / (t128_13 * 1e-6) / 1e12
    f128_2 = 2.0 * 128 * 2048 * 8192 / (t128_2 * 1e-6) / 1e12
    # the prompt window over two alternating copies of weights and prompt
    xw = to_dev(synthetic.draw_bf16_rows(rng, 8192, 2048), np.int16, dev).view(torch.bfloat16)
    wins = [(pool[0][0], pool[0][1], xw), (pool[1][0], pool[1][1], xw.clone())]
    zw = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    tw = graph_us(torch, lambda i: win_call(wins[i % 2][0], wins[i % 2][1], wins[i % 2][2], zw), 6)
    tf = 2.0 * 8192 * (2 * 8192) * 2048 / (tw * 1e-6) / 1e12
    del pool, wins, zw, xw
    torch.cuda.empty_cache()
    return {
        "decode_step": {"us": r3(t_step), "GB/s": round((b13 + b2) / (t_step * 1e-6) / 1e9, 1)},
        "qmv_w13_swiglu": {"us": r3(t13), "frac": round(b13 / (t13 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "qmv_rows_w2_f32x": {"us": r3(t2), "frac": round(b2 / (t2 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "pgemm_swiglu_8192": {"us": r3(tw), "TFLOP/s": round(tf, 2), "frac": round(tf / BF16_PEAK_TFLOPS, 4)},
        "window_128": {"w1w3_swiglu": {"us": r3(t128_13), "TFLOP/s": round(f128_13, 2)},
                       "w2": {"us": r3(t128_2), "TFLOP/s": round(f128_2, 2)}},
    }


# HBM bytes the 8192-row w1/w3 + SwiGLU window must move at least: both
# packed weights once, the bf16 prompt once, the bf16 output once
PGEMM_BYTES = 2 * (8192 * 2048 * 9 // 16) + 8192 * 2048 * 2 + 8192 * 8192 * 2


def pgemm_only(dev, reps=6):
    """Only the 8192-row w1/w3 + SwiGLU window (bf16 out), on two alternating
    copies of weights and prompt: the dispatches the prompt GEMM's counters
    are taken on."""
    import torch

    import bit_weight_only_q4g64_amd as q4
    import synthetic

    rng = np.random.default_rng(4)
    w1, w3 = synthetic.draw_qweight(rng, "w1", 8192, 2048), synthetic.draw_qweight(rng, "w3", 8192, 2048)
    xh = synthetic.draw_bf16_rows(rng, 8192, 2048)
    copies = [(pack_dev(w1, dev), pack_dev(w3, dev), to_dev(xh, np.int16, dev).view(torch.bfloat16)) for _ in range(2)]
    z = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
    ts = []
    for r in range(reps):
        p1, p3, x = copies[r % 2]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        q4.qmm_window(p1, p3, 8192, 2048, x, y=z)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    t = float(np.median(ts[1:]))
    return {"avg_us": round(t * 1e6, 2), "TFLOP/s": round(2.0 * 8192 * 16384 * 2048 / t / 1e12, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true", help="only the headline decode step (for its per-dispatch counters)")
    ap.add_argument("--no-wide", action="store_true", help="skip the 6-/8-bit, block-FP8 and attention-epilogue measurements")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps directly instead of replaying a graph (for per-dispatch counters)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (the reference for scaling HBM byte counters)")
    ap.add_argument("--pgemm-only", action="store_true",
                    help="only the 8192-row w1/w3 + SwiGLU window (for its per-dispatch counters); prints its JSON object")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the machines this runs on have one, and the multi-GPU path is a design only "
              "(sharding over output columns for decode and over prompt rows for windows)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return
    import bit_weight_only_q4g64_amd as q4
    import synthetic

    q4.lib()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.pgemm_only:
        print(json.dumps(pgemm_only(dev)))
        return

    log("generating the decode FFN workload")
    d = synthetic.config(1)
    K, W = args.steps, args.warmup
    st = bench_step(d, dev, K, W, no_graph=args.no_graph)
    step_bytes = decode_step_bytes(d)
    value = step_bytes / (st["ms_per_step"] * 1e-3) / 1e9
    kernel_gbs = step_bytes / (st["step_kernel_us"] * 1e-6) / 1e9
    w1, w2 = d["w1"], d["w2"]
    b13 = 2 * qbytes(w1.N, w1.K) + w1.K * 2 + w1.N * 4
    b2 = qbytes(w2.N, w2.K) + w2.K * 4 + w2.N * 4
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(st["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode FFN step: z = silu(W1 x) * (W3 x) over w1/w3 8192x2048 q4g64, then y = W2 z over w2 2048x8192 "
                        "q4g64 on the float32 z, as one qmv_ffn launch; 1 bf16 activation row; seed 1",
            "rows": 1,
            "step_bytes": step_bytes,
            "weight_pool_copies": st["pool_copies"],
            "timing": ("HIP graph of K steps" if not args.no_graph else "K directly launched steps")
            + "; value from the wall clock between synchronizes, kernel time from HIP events around the same region",
        },
        "rows_per_s": round(1.0 / (st["ms_per_step"] * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "kernel": "q4::ffn_flow_kernel<1, 1> (qmv_ffn, the whole step in one launch)",
            "achieved": round(kernel_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic_per_launch("ffn_flow_step"),
            "algorithmic_bytes_per_launch": step_bytes,
            "avg_launch_us": round(st["step_kernel_us"], 3),
            "step_frac": round(value / HBM_PEAK_GBS, 4),
            "kernels": {
                "ffn_flow_step": {"us": r3(st["ffn_graph_us"]), "bytes": step_bytes,
                                  "frac": round(step_bytes / (st["ffn_graph_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
                "two_calls_step": {"us": r3(st["two_calls_us"]), "bytes": step_bytes,
                                   "frac": round(step_bytes / (st["two_calls_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
                "qmv_w13_swiglu": {"us": r3(st["w13_us"]), "bytes": b13, "frac": round(b13 / (st["w13_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                   "traffic": traffic_per_launch("qmv_w13_swiglu")},
                "qmv_rows_w2_f32x": {"us": r3(st["w2_us"]), "bytes": b2, "frac": round(b2 / (st["w2_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                     "traffic": traffic_per_launch("qmv_rows_w2")},
            },
            "target": "0.70 of the HBM peak for decode (28.4 MB in <= 5.1 us)",
        },
    }
    if args.step_only:
        print(json.dumps(result), flush=True)
        return
    inputs = {"c1": input_hashes(d)}
    log("c0 single matvec")
    result["c0"] = bench_c0(dev, K)
    log("c2 attention projections")
    result["c2"] = bench_c2(dev, K)
    log("c3 1000-row prompt cuts")
    result["c3"] = bench_c3(dev, K)
    result["c4"] = bench_c4(dev)
    inputs["c4"] = result["c4"].pop("inputs_sha256")
    w13 = result["c4"]["whole"]["w1w3_swiglu"]
    result["pgemm"] = {
        "workload": "the 8192-row layer's w1/w3 + SwiGLU window (bf16 out), the largest window of the layer",
        "roofline": {"bound": "mfma", "kernel": "q4::pgemm_kernel<true, true, 4>", "achieved": w13["TFLOP/s"],
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": w13["frac"],
                     "traffic": traffic_per_launch("pgemm_swiglu_8192"), "algorithmic_bytes_per_launch": PGEMM_BYTES,
                     "avg_launch_us": w13["us"], "mfma_counters": summary_json("mfma_pgemm_swiglu_8192.md"),
                     "target": "0.50 of the bf16 matrix-core peak"},
    }
    log("decode step at 1..16 rows")
    result["decode_rows"] = bench_rows(dev, K)
    result["rows_per_s_at_16_rows"] = result["decode_rows"]["R16"]["best_rows_per_s"]
    if not args.no_wide:
        log("attention epilogue")
        result["qkv_rope"] = bench_qkv_rope(dev, K)
        log("6-bit, 8-bit and block-FP8 weights")
        result["wide_codes"] = {str(b): bench_wide(dev, b, K) for b in (6, 8, "fp8")}
    result["copy_bandwidth"] = copy_bandwidth(torch)
    for i in (0, 2, 3):
        inputs[f"c{i}"] = input_hashes(synthetic.config(i))
    result["provenance"] = provenance(torch, inputs)
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host")
        result["cpu_baseline"] = cpu_baseline(d, st["z"], st["y"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
