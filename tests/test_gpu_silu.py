"""FP64 op test of the device SwiGLU gate (TensorFold PR #1696, "What it
adds" > Kernels without DPAS: an FP64 op test and a planted control per
kernel; the planted control is test_silu_model.py's single-float exponent).

A one-hot activation and one-group weights make every output column's gate
argument a = fl32(s * q + b), formed here from the column's (s, q, b), with
c = 1 from a second weight (scale 0, bias 1). The decode matvec and the
prompt window must produce exactly that a, and their fused SwiGLU outputs
silu(a) * 1 must lie within the stated bound of the float64 silu at a."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import oracle
from tests import silu_cases
from tests.gpu_helpers import bits32, dev_bf16, dev_weight, host_f64, say
from tests.test_silu_model import case_arguments, excess

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def silu_dev():
    wa, wc, x = silu_cases.weights()
    return {"wa": wa, "pa": dev_weight(wa), "pc": dev_weight(wc), "x": dev_bf16(x), "a": case_arguments()}


def _check(a_dev, z_dev, a, label):
    assert np.array_equal(bits32(a_dev)[0], a.view(np.int32)), f"{label}: gate arguments differ from fl32(s*q + b)"
    z = host_f64(z_dev)[0].astype(np.float32)
    r = excess(z, a)
    say(f"{label}: max |silu_dev - silu64| / bound = {r:.3g}")
    assert r <= 1.0, f"{label}: {r}"


def test_decode_silu_within_bound(silu_dev):
    N = silu_dev["wa"].N
    say(f"device silu via qmv_w13_swiglu, {N} arguments")
    a_dev = q4.qmv_rows(silu_dev["pa"], N, silu_cases.K, silu_dev["x"])
    z_dev = q4.qmv_w13_swiglu(silu_dev["pa"], silu_dev["pc"], N, silu_cases.K, silu_dev["x"])
    torch.cuda.synchronize()
    _check(a_dev, z_dev, silu_dev["a"], "decode")


def test_window_silu_within_bound(silu_dev):
    N = silu_dev["wa"].N
    say(f"device silu via the qmm_window SwiGLU epilogue, {N} arguments")
    x2 = silu_dev["x"].repeat(3, 1)  # three identical rows: the epilogue of every row slot
    a_dev = q4.qmm_window(silu_dev["pa"], None, N, silu_cases.K, x2)
    z_dev = q4.qmm_window(silu_dev["pa"], silu_dev["pc"], N, silu_cases.K, x2)
    torch.cuda.synchronize()
    for r in range(3):
        _check(a_dev[r : r + 1], z_dev[r : r + 1], silu_dev["a"], f"window row {r}")
