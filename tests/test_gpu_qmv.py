"""Decode matvecs on the GPU against the float64 oracle, plus the bit
invariances: N-row equals 1-row, row permutation, strides, run-to-run."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import oracle
import synthetic
from tests.gpu_helpers import DEV, bits32, check_within, dev_bf16, dev_f32, dev_weight, host_f64, say
from tests.tolerance import tol, tol_swiglu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c2():
    d = synthetic.config(2)
    d["qkv"] = synthetic.concat_rows(d["wq"], d["wk"], d["wv"], name="qkv")
    d["p_qkv"] = dev_weight(d["qkv"])
    d["p_o"] = dev_weight(d["wo"])
    d["xd"] = dev_bf16(d["x"])
    return d


def test_c0_single_matvec():
    d = synthetic.config(0)
    w = d["w"]
    say("c0 qmv_rows N=512 K=256 R=1")
    y = q4.qmv_rows(dev_weight(w), w.N, w.K, dev_bf16(d["x"]))
    torch.cuda.synchronize()
    r, ra = check_within(host_f64(y), w, d["x"], label="c0", order="decode")
    say(f"c0 max err/T {r:.3g} max err/A {ra:.3g}")


@pytest.mark.parametrize("R", [1, 2, 4, 8, 16])
def test_c2_attention_projections(c2, R):
    say(f"c2 qkv/o R={R}")
    for name, pk in (("qkv", "p_qkv"), ("wo", "p_o")):
        w = c2[name]
        y = q4.qmv_rows(c2[pk], w.N, w.K, c2["xd"][:R])
        torch.cuda.synchronize()
        check_within(host_f64(y), w, c2["x"][:R], label=f"c2 {name} R={R}", order="decode")


def test_c2_rows_bit_equal_to_one_row(c2):
    say("c2 N-row vs 1-row bits")
    for name, pk in (("qkv", "p_qkv"), ("wo", "p_o")):
        w = c2[name]
        ones = [bits32(q4.qmv_rows(c2[pk], w.N, w.K, c2["xd"][r : r + 1])) for r in range(16)]
        for R in (2, 3, 4, 5, 8, 11, 16):
            yR = bits32(q4.qmv_rows(c2[pk], w.N, w.K, c2["xd"][:R]))
            for r in range(R):
                assert np.array_equal(yR[r], ones[r][0]), (name, R, r)


def test_c2_row_permutation_and_strides(c2):
    say("c2 row permutation / padded stride")
    w = c2["qkv"]
    perm = np.random.default_rng(5).permutation(16)
    y = bits32(q4.qmv_rows(c2["p_qkv"], w.N, w.K, c2["xd"]))
    yp = bits32(q4.qmv_rows(c2["p_qkv"], w.N, w.K, c2["xd"][torch.from_numpy(perm).to(DEV)]))
    assert np.array_equal(yp, y[perm])
    # x rows with a padded stride and y with a padded stride
    xpad = torch.zeros((16, w.K + 64), dtype=torch.bfloat16, device=DEV)
    xpad[:, : w.K] = c2["xd"]
    ybuf = torch.full((16, w.N + 32), float("nan"), device=DEV)
    q4.qmv_rows(c2["p_qkv"], w.N, w.K, xpad[:, : w.K], y=ybuf[:, : w.N])
    torch.cuda.synchronize()
    assert np.array_equal(bits32(ybuf[:, : w.N]), y)
    assert torch.isnan(ybuf[:, w.N :]).all()  # nothing written past N


def test_c2_deterministic(c2):
    w = c2["wo"]
    a = bits32(q4.qmv_rows(c2["p_o"], w.N, w.K, c2["xd"]))
    b = bits32(q4.qmv_rows(c2["p_o"], w.N, w.K, c2["xd"]))
    assert np.array_equal(a, b)


def test_c1_fused_w13_swiglu():
    d = synthetic.config(1)
    w1, w3 = d["w1"], d["w3"]
    say("c1 qmv_w13_swiglu N=8192 K=2048 R=1")
    p1, p3 = dev_weight(w1), dev_weight(w3)
    z = host_f64(q4.qmv_w13_swiglu(p1, p3, w1.N, w1.K, dev_bf16(d["x"])))
    a64 = oracle.matmul_rows(w1.wq, w1.scales, w1.biases, d["x"])
    c64 = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, d["x"])
    Ta = tol(oracle.error_weight(w1.wq, w1.scales, w1.biases, d["x"]), w1.K, order="decode")
    Tc = tol(oracle.error_weight(w3.wq, w3.scales, w3.biases, d["x"]), w3.K, order="decode")
    z64 = oracle.swiglu(a64, c64)
    Tz = tol_swiglu(a64, c64, Ta, Tc)
    ratio = float(np.max(np.abs(z - z64) / Tz))
    say(f"c1 swiglu max err/Tz {ratio:.3g}")
    assert ratio <= 1.0


def test_c1_fused_rows_bit_equal_to_one_row():
    d = synthetic.config(1)
    w1, w3 = d["w1"], d["w3"]
    p1, p3 = dev_weight(w1), dev_weight(w3)
    rng = np.random.default_rng(9)
    x = dev_bf16(synthetic.draw_bf16_rows(rng, 16, w1.K))
    z16 = bits32(q4.qmv_w13_swiglu(p1, p3, w1.N, w1.K, x))
    for r in (0, 5, 15):
        z1 = bits32(q4.qmv_w13_swiglu(p1, p3, w1.N, w1.K, x[r : r + 1]))
        assert np.array_equal(z16[r], z1[0]), r


def test_c1_w2_float32_input():
    """w2 consumes a float32 input (the SwiGLU output) unrounded."""
    d = synthetic.config(1)
    w2 = d["w2"]
    say("c1 w2 float32 x N=2048 K=8192")
    p2 = dev_weight(w2)
    x = d["x_w2_f32"]
    y = host_f64(q4.qmv_rows(p2, w2.N, w2.K, dev_f32(x)))
    r, _ = check_within(y, w2, x, x_dtype="f32", label="c1 w2 f32", order="decode")
    y1 = bits32(q4.qmv_rows(p2, w2.N, w2.K, dev_f32(x[2:3])))
    y4 = bits32(q4.qmv_rows(p2, w2.N, w2.K, dev_f32(x)))
    assert np.array_equal(y4[2], y1[0])


def test_c1_decode_chain_against_float64_chain():
    """GPU w13+SwiGLU (float32) -> GPU w2, against the oracle's float64 chain,
    with the SwiGLU bound propagated through |W2|."""
    d = synthetic.config(1)
    w1, w3, w2 = d["w1"], d["w3"], d["w2"]
    say("c1 decode chain")
    z = q4.qmv_w13_swiglu(dev_weight(w1), dev_weight(w3), w1.N, w1.K, dev_bf16(d["x"]))
    y2 = host_f64(q4.qmv_rows(dev_weight(w2), w2.N, w2.K, z))
    a64 = oracle.matmul_rows(w1.wq, w1.scales, w1.biases, d["x"])
    c64 = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, d["x"])
    z64 = oracle.swiglu(a64, c64)
    Tz = tol_swiglu(a64, c64, tol(oracle.error_weight(w1.wq, w1.scales, w1.biases, d["x"]), w1.K, order="decode"),
                    tol(oracle.error_weight(w3.wq, w3.scales, w3.biases, d["x"]), w3.K, order="decode"))
    y64 = oracle.matmul_rows(w2.wq, w2.scales, w2.biases, z64)
    bound = tol(oracle.error_weight(w2.wq, w2.scales, w2.biases, np.abs(z64) + Tz), w2.K, "f32", order="decode") + \
        oracle.error_weight(w2.wq, w2.scales, w2.biases, Tz)
    ratio = float(np.max(np.abs(y2 - y64) / bound))
    say(f"c1 chain max err/bound {ratio:.3g}")
    assert ratio <= 1.0


@pytest.mark.parametrize("N,K,R", [(64, 64, 1), (64, 192, 3), (128, 640, 7), (64, 16384, 16), (256, 1024, 16)])
def test_edge_shapes_signed_scales(N, K, R):
    """Odd group counts, a partial last segment, the maximum decode K, and
    scales of every sign (zero included) with activations over a wide range."""
    say(f"edge qmv N={N} K={K} R={R}")
    rng = np.random.default_rng(N + K + R)
    w = synthetic.draw_qweight(rng, "edge", N, K)
    s = (w.scales.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s *= rng.choice([-1.0, 1.0, 0.0, 300.0], size=s.shape, p=[0.3, 0.5, 0.1, 0.1])
    w.scales = synthetic.bf16_bits_from_f64(s)
    x = synthetic.bf16_bits_from_f64(rng.normal(0, 1, (R, K)) * rng.choice([1e-4, 1.0, 50.0], (R, K)))
    pk = dev_weight(w)
    y = host_f64(q4.qmv_rows(pk, N, K, dev_bf16(x)))
    check_within(y, w, x, label=f"edge {N}x{K} R={R}", order="decode")
    xf = (rng.normal(0, 1, (R, K)) * rng.choice([1e-3, 1.0, 30.0], (R, K))).astype(np.float32)
    yf = host_f64(q4.qmv_rows(pk, N, K, dev_f32(xf)))
    check_within(yf, w, xf, x_dtype="f32", label=f"edge f32 {N}x{K} R={R}", order="decode")


def test_zero_activations_give_zero():
    w = synthetic.config(0)["w"]
    y = q4.qmv_rows(dev_weight(w), w.N, w.K, torch.zeros((3, w.K), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("R", [1, 3, 16])
def test_two_tile_workgroups_keep_the_columns(bits, R):
    """A one-matrix bf16 matvec over at least 512 column tiles runs two column tiles per workgroup. Its columns
    equal, bit for bit, the same columns computed by the one-tile kernel on a narrower matrix made of the same
    rows (the first 1024 rows of an 8192-row matrix, packed on their own), and every row equals its one-row call."""
    say(f"two-tile workgroups bits={bits} R={R}")
    rng = np.random.default_rng(1200 + bits + R)
    N, K, n = 8192, 2048, 1024
    w = synthetic.draw_qweight(rng, "w", N, K, bits=bits)
    part = synthetic.QWeight("w_head", n, K, w.wq[:n].copy(), w.scales[:n].copy(), w.biases[:n].copy(), bits)
    x = dev_bf16(synthetic.draw_bf16_rows(rng, R, K))
    y = q4.qmv_rows(dev_weight(w), N, K, x, bits=bits)
    yp = q4.qmv_rows(dev_weight(part), n, K, x, bits=bits)
    torch.cuda.synchronize()
    assert np.array_equal(bits32(y)[:, :n], bits32(yp))
    y1 = q4.qmv_rows(dev_weight(w), N, K, x[R - 1 : R], bits=bits)
    torch.cuda.synchronize()
    assert np.array_equal(bits32(y1)[0], bits32(y)[R - 1])
