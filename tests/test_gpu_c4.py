"""The long-prompt layer at full size: 8192 rows through qkv, o, w1/w3 with
SwiGLU (bf16 out), w2 on that bf16 output, and the 65536 x 2048 head on the
last 128 rows. Parity on sampled outputs the oracle computes one by one, and
bit-identity between the whole prompt as one window and 128-row windows."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import oracle
import synthetic
from tests.gpu_helpers import DEV, bits16, bits32, check_within, dev_bf16, dev_weight, host_f64, say
from tests.tolerance import tol, tol_bf16_out, tol_swiglu

pytestmark = pytest.mark.gpu

ROWS = [0, 1, 127, 128, 129, 1000, 4095, 4096, 6000, 8190, 8191]


@pytest.fixture(scope="module")
def c4():
    say("c4 generating inputs")
    d = synthetic.config(4)
    d["qkv"] = synthetic.concat_rows(d["wq"], d["wk"], d["wv"], name="qkv")
    for name in ("qkv", "wo", "w1", "w3", "w2", "head"):
        d["p_" + name] = dev_weight(d[name])
    d["xd"] = dev_bf16(d["x"])
    torch.cuda.synchronize()
    return d


def test_c4_qkv_and_o(c4):
    for name in ("qkv", "wo"):
        w = c4[name]
        say(f"c4 {name} M=8192")
        y = q4.qmm_window(c4["p_" + name], None, w.N, w.K, c4["xd"])
        torch.cuda.synchronize()
        check_within(host_f64(y[ROWS]), w, c4["x"], rows=ROWS, label=f"c4 {name}", order="window")
        if name == "qkv":
            yc = q4.qmm_cut(c4["p_" + name], None, w.N, w.K, c4["xd"], [128] * 64)
            torch.cuda.synchronize()
            assert np.array_equal(bits32(yc), bits32(y))


def test_c4_ffn_chain(c4):
    w1, w3, w2 = c4["w1"], c4["w3"], c4["w2"]
    say("c4 w1/w3 SwiGLU bf16 M=8192")
    z = q4.qmm_window(c4["p_w1"], c4["p_w3"], w1.N, w1.K, c4["xd"], out_dtype=torch.bfloat16)
    zc = q4.qmm_cut(c4["p_w1"], c4["p_w3"], w1.N, w1.K, c4["xd"], [128] * 64, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(zc), bits16(z))
    xs = c4["x"][ROWS]
    a64 = oracle.matmul_rows(w1.wq, w1.scales, w1.biases, xs)
    c64 = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, xs)
    z64 = oracle.swiglu(a64, c64)
    Tz = tol_swiglu(a64, c64, tol(oracle.error_weight(w1.wq, w1.scales, w1.biases, xs), w1.K, order="window"),
                    tol(oracle.error_weight(w3.wq, w3.scales, w3.biases, xs), w3.K, order="window"))
    Ez = tol_bf16_out(z64, Tz)
    zg = oracle.bf16_to_f64(bits16(z[ROWS]).view(np.uint16))
    assert np.all(np.abs(zg - z64) <= Ez)
    say("c4 w2 on the bf16 SwiGLU output")
    y2 = q4.qmm_window(c4["p_w2"], None, w2.N, w2.K, z)
    torch.cuda.synchronize()
    y64 = oracle.matmul_rows(w2.wq, w2.scales, w2.biases, z64)
    bound = tol(oracle.error_weight(w2.wq, w2.scales, w2.biases, np.abs(z64) + Ez), w2.K, order="window") + \
        oracle.error_weight(w2.wq, w2.scales, w2.biases, Ez)
    assert np.all(np.abs(host_f64(y2[ROWS]) - y64) <= bound)


def test_c4_w2_standalone_bf16_input(c4):
    w2 = c4["w2"]
    say("c4 w2 per-op parity on the bf16 stand-in input")
    x = c4["x_w2_bf16"]
    y = q4.qmm_window(c4["p_w2"], None, w2.N, w2.K, dev_bf16(x))
    torch.cuda.synchronize()
    check_within(host_f64(y[:24]), w2, x[:24], label="c4 w2", order="window")


def test_c4_head_last_128_rows(c4):
    w = c4["head"]
    say("c4 head N=65536 on the last 128 rows")
    xl = c4["xd"][-128:]
    y = q4.qmm_window(c4["p_head"], None, w.N, w.K, xl)
    torch.cuda.synchronize()
    cols = np.random.default_rng(4).choice(w.N, 1024, replace=False)
    rows = [0, 63, 64, 127]
    yg = host_f64(y[rows])[:, cols]
    check_within(yg, w, c4["x"][-128:][rows], cols=cols, label="c4 head", order="window")
    # row 8191 of the prompt computed alone equals row 127 of the head window
    y1 = q4.qmm_window(c4["p_head"], None, w.N, w.K, xl[127:128])
    assert np.array_equal(bits32(y1)[0], bits32(y)[127])
