"""Helpers shared by the GPU tests: move canonical numpy tensors to the device
and compare GPU results with the oracle under the stated bounds."""

import sys

import numpy as np
import torch

import bit_weight_only_q4g64_amd as q4
import oracle
from tests.tolerance import tol

DEV = "cuda:0"


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def dev_weight(w):
    """Canonical QWeight -> packed device tensor."""
    wq = torch.from_numpy(np.ascontiguousarray(w.wq).view(np.int32)).to(DEV)
    sc = torch.from_numpy(np.ascontiguousarray(w.scales).view(np.int16)).to(DEV)
    bi = torch.from_numpy(np.ascontiguousarray(w.biases).view(np.int16)).to(DEV)
    return q4.pack(wq, sc, bi, bits=getattr(w, "bits", 4))


def dev_bf16(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits32(t):
    return t.detach().contiguous().view(torch.int32).cpu().numpy()


def bits16(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy()


def check_within(y_gpu, w, x, cols=None, x_dtype="bf16", rows=None, label="", *, order):
    """|y_gpu - y64| <= T elementwise, T for the kernel family ``order``
    (decode or window); returns (max err/T, max err/A)."""
    xs = x if rows is None else x[rows]
    bits = getattr(w, "bits", 4)
    y64 = oracle.matmul_rows(w.wq, w.scales, w.biases, xs, cols=cols, bits=bits)
    A = oracle.error_weight(w.wq, w.scales, w.biases, xs, cols=cols, bits=bits)
    T = tol(A, w.K, x_dtype, order=order)
    err = np.abs(y_gpu - y64)
    ratio = float(np.max(err / T))
    assert np.all(np.isfinite(y_gpu)), label
    assert ratio <= 1.0, f"{label}: max |err|/T = {ratio}"
    return ratio, float(np.max(err / A))
