"""Accuracy figures of every workload against the float64 oracle (TensorFold
PR #1696, "Checks" > Forward against float64: error as a multiple of the
bf16 gap; later revision, "Checks" > pgemm against float64: float32 error and
bf16 flips). Reported, not gated: the gate is the stated bound in the parity
tests. Each case prints one line; the whole table is written to
gpurun_out/accuracy.json when that folder exists."""

import json
import os

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import oracle
import synthetic
from oracle.diagnostics import accuracy
from tests.gpu_helpers import dev_bf16, dev_weight, host_f64, say

pytestmark = pytest.mark.gpu

TABLE = {}


def _report(name, y, y64, A):
    a = accuracy(y, y64, A)
    TABLE[name] = a
    say(f"accuracy {name}: bf16-gap ratio {a['bf16_gap_ratio']:.3g}, flips {a['bf16_flips']}/{a['outputs']}, "
        f"max err/A {a['max_err_over_A']:.3g}, RMS err/A {a['rms_err_over_A']:.3g}")
    if os.path.isdir("gpurun_out"):
        with open(os.path.join("gpurun_out", "accuracy.json"), "w") as f:
            json.dump(TABLE, f, indent=1)
    assert np.all(np.isfinite(y))


def test_c0():
    d = synthetic.config(0)
    w = d["w"]
    y = host_f64(q4.qmv_rows(dev_weight(w), w.N, w.K, dev_bf16(d["x"])))
    _report("c0 qmv_rows", y, oracle.matmul_rows(w.wq, w.scales, w.biases, d["x"]), oracle.error_weight(w.wq, w.scales, w.biases, d["x"]))


def test_c1_step():
    d = synthetic.config(1)
    w1, w3, w2 = d["w1"], d["w3"], d["w2"]
    work = q4.ffn_workspace(w1.N, w2.N, 1, "cuda:0")
    z, y = q4.qmv_ffn(dev_weight(w1), dev_weight(w3), dev_weight(w2), w1.N, w1.K, w2.N, dev_bf16(d["x"]), work)
    torch.cuda.synchronize()
    a64 = oracle.matmul_rows(w1.wq, w1.scales, w1.biases, d["x"])
    c64 = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, d["x"])
    z64 = oracle.swiglu(a64, c64)
    Az = np.abs(oracle.silu(a64)) * oracle.error_weight(w3.wq, w3.scales, w3.biases, d["x"]) + \
        np.abs(c64) * oracle.error_weight(w1.wq, w1.scales, w1.biases, d["x"])
    _report("c1 z (qmv_ffn)", host_f64(z), z64, Az)
    y64 = oracle.matmul_rows(w2.wq, w2.scales, w2.biases, z64)
    _report("c1 y (qmv_ffn, float64 chain)", host_f64(y), y64, oracle.error_weight(w2.wq, w2.scales, w2.biases, np.abs(z64)))


@pytest.mark.parametrize("R", [1, 16])
def test_c2(R):
    d = synthetic.config(2)
    qkv = synthetic.concat_rows(d["wq"], d["wk"], d["wv"], name="qkv")
    x = d["x"][:R]
    for name, w in (("qkv", qkv), ("o", d["wo"])):
        y = host_f64(q4.qmv_rows(dev_weight(w), w.N, w.K, dev_bf16(x)))
        _report(f"c2 {name} R={R}", y, oracle.matmul_rows(w.wq, w.scales, w.biases, x), oracle.error_weight(w.wq, w.scales, w.biases, x))


def test_c3_window():
    d = synthetic.config(3)
    w1, w3 = d["w1"], d["w3"]
    rows = [0, 17, 316, 999]
    a = host_f64(q4.qmm_window(dev_weight(w1), None, w1.N, w1.K, dev_bf16(d["x"])))[rows]
    xs = d["x"][rows]
    _report("c3 w1 window rows 0/17/316/999", a, oracle.matmul_rows(w1.wq, w1.scales, w1.biases, xs),
            oracle.error_weight(w1.wq, w1.scales, w1.biases, xs))
    del w3


def test_c4_head():
    d = synthetic.config(4, rows=256)
    w = d["head"]
    xl = d["x"][-128:]
    y = host_f64(q4.qmm_window(dev_weight(w), None, w.N, w.K, dev_bf16(xl)))[[0, 127]]
    xs = xl[[0, 127]]
    _report("c4 head rows 0/127", y, oracle.matmul_rows(w.wq, w.scales, w.biases, xs), oracle.error_weight(w.wq, w.scales, w.biases, xs))
