"""Block-FP8 weight-only weights (PR #1696: the block FP8 export served
weight-only) through the same boundary: pack bit-exact against the layout
model and invertible; decode and window results within the stated tolerance
of the float64 oracle; N-row = 1-row, cut and single-row bit rules."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import oracle
import synthetic
from tests.gpu_helpers import DEV, bits32, dev_bf16, dev_f32, host_f64, say
from tests.layout_model import pack_model_fp8
from tests.tolerance import tol, tol_swiglu

pytestmark = pytest.mark.gpu


def dev_fp8(w):
    return q4.pack_fp8b(torch.from_numpy(np.ascontiguousarray(w.w8)).to(DEV), torch.from_numpy(np.ascontiguousarray(w.scales)).to(DEV))


def check_fp8(y, w, x, cols=None, x_dtype="bf16", label="", *, order):
    """|y - y64| <= T elementwise on the sampled columns."""
    y64 = oracle.matmul_rows_fp8(w.w8, w.scales, x, cols=cols)
    T = tol(oracle.error_weight_fp8(w.w8, w.scales, x, cols=cols), w.K, x_dtype, order=order, fmt="fp8")
    r = float(np.max(np.abs(y - y64) / T))
    assert np.all(np.isfinite(y)), label
    assert r <= 1.0, f"{label}: max err/T {r}"
    return r


@pytest.mark.parametrize("N,K", [(64, 64), (192, 192), (256, 640), (128, 2048)])
def test_fp8_pack_bit_exact_and_invertible(N, K):
    say(f"pack_fp8b N={N} K={K}")
    w = synthetic.draw_fp8_weight(np.random.default_rng(N + 3 * K), "w", N, K)
    p = dev_fp8(w)
    torch.cuda.synchronize()
    assert p.numel() == q4.fp8b_packed_bytes(N, K)
    assert np.array_equal(p.cpu().numpy(), pack_model_fp8(w.w8, w.scales, N, K))
    w8, sc = q4.unpack_fp8b(p, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(w8.cpu().numpy(), w.w8)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), w.scales.view(np.uint32))


@pytest.fixture(scope="module")
def fp8():
    rng = np.random.default_rng(700)
    d = {}
    d["qkv"] = synthetic.draw_fp8_weight(rng, "qkv", 3072, 2048)
    d["w2"] = synthetic.draw_fp8_weight(rng, "w2", 2048, 8192)
    d["w1"] = synthetic.draw_fp8_weight(rng, "w1", 1024, 2048)
    d["w3"] = synthetic.draw_fp8_weight(rng, "w3", 1024, 2048)
    d["x"] = synthetic.draw_bf16_rows(rng, 16, 2048)
    d["xf"] = synthetic.draw_f32_rows(rng, 8, 8192, sigma=0.05)
    for k in ("qkv", "w2", "w1", "w3"):
        d["p_" + k] = dev_fp8(d[k])
    return d


@pytest.mark.parametrize("R", [1, 3, 16])
def test_fp8_qmv_bf16_within_tolerance(fp8, R):
    w = fp8["qkv"]
    say(f"qmv_rows_fp8b {w.N}x{w.K} R={R}")
    y = q4.qmv_rows_fp8b(fp8["p_qkv"], w.N, w.K, dev_bf16(fp8["x"][:R]))
    torch.cuda.synchronize()
    cols = np.arange(0, w.N, 5)
    check_fp8(host_f64(y)[:, cols], w, fp8["x"][:R], cols=cols, label=f"fp8 R={R}", order="decode")


@pytest.mark.parametrize("R", [1, 5])
def test_fp8_qmv_f32_within_tolerance(fp8, R):
    w = fp8["w2"]
    say(f"qmv_rows_fp8b f32 x {w.N}x{w.K} R={R}")
    y = q4.qmv_rows_fp8b(fp8["p_w2"], w.N, w.K, dev_f32(fp8["xf"][:R]))
    torch.cuda.synchronize()
    cols = np.arange(1, w.N, 3)
    check_fp8(host_f64(y)[:, cols], w, fp8["xf"][:R], cols=cols, x_dtype="f32", label=f"fp8 f32 R={R}", order="decode")


def test_fp8_rows_bit_equal_to_one_row(fp8):
    w = fp8["qkv"]
    xd = dev_bf16(fp8["x"])
    yR = bits32(q4.qmv_rows_fp8b(fp8["p_qkv"], w.N, w.K, xd))
    for r in (0, 5, 15):
        assert np.array_equal(yR[r], bits32(q4.qmv_rows_fp8b(fp8["p_qkv"], w.N, w.K, xd[r : r + 1]))[0]), r
    w2 = fp8["w2"]
    xf = dev_f32(fp8["xf"])
    yR = bits32(q4.qmv_rows_fp8b(fp8["p_w2"], w2.N, w2.K, xf))
    for r in (0, 7):
        assert np.array_equal(yR[r], bits32(q4.qmv_rows_fp8b(fp8["p_w2"], w2.N, w2.K, xf[r : r + 1]))[0]), r


@pytest.mark.parametrize("R", [1, 4])
def test_fp8_w13_swiglu(fp8, R):
    w1, w3 = fp8["w1"], fp8["w3"]
    say(f"qmv_w13_swiglu_fp8b R={R}")
    xs = fp8["x"][:R]
    z = q4.qmv_w13_swiglu_fp8b(fp8["p_w1"], fp8["p_w3"], w1.N, w1.K, dev_bf16(xs))
    torch.cuda.synchronize()
    a64 = oracle.matmul_rows_fp8(w1.w8, w1.scales, xs)
    c64 = oracle.matmul_rows_fp8(w3.w8, w3.scales, xs)
    Tz = tol_swiglu(a64, c64, tol(oracle.error_weight_fp8(w1.w8, w1.scales, xs), w1.K, order="decode", fmt="fp8"),
                    tol(oracle.error_weight_fp8(w3.w8, w3.scales, xs), w3.K, order="decode", fmt="fp8"))
    assert np.all(np.abs(host_f64(z) - oracle.swiglu(a64, c64)) <= Tz)


WIN_ROWS = [0, 1, 63, 64, 127, 128, 255, 256, 299, 300, 449]


@pytest.fixture(scope="module")
def fp8_win():
    rng = np.random.default_rng(710)
    d = {"a": synthetic.draw_fp8_weight(rng, "a", 1024, 2112), "b": synthetic.draw_fp8_weight(rng, "b", 1024, 2112)}
    d["x"] = synthetic.draw_bf16_rows(rng, 450, 2112)
    d["pa"], d["pb"], d["xd"] = dev_fp8(d["a"]), dev_fp8(d["b"]), dev_bf16(d["x"])
    d["plain"] = q4.qmm_window_fp8b(d["pa"], None, 1024, 2112, d["xd"])
    d["swiglu"] = q4.qmm_window_fp8b(d["pa"], d["pb"], 1024, 2112, d["xd"])
    torch.cuda.synchronize()
    return d


def test_fp8_window_parity(fp8_win):
    a, b = fp8_win["a"], fp8_win["b"]
    xs = fp8_win["x"][WIN_ROWS]
    say("qmm_window_fp8b parity")
    check_fp8(host_f64(fp8_win["plain"])[WIN_ROWS], a, xs, label="fp8 window", order="window")
    a64 = oracle.matmul_rows_fp8(a.w8, a.scales, xs)
    c64 = oracle.matmul_rows_fp8(b.w8, b.scales, xs)
    Tz = tol_swiglu(a64, c64, tol(oracle.error_weight_fp8(a.w8, a.scales, xs), a.K, order="window", fmt="fp8"),
                    tol(oracle.error_weight_fp8(b.w8, b.scales, xs), b.K, order="window", fmt="fp8"))
    assert np.all(np.abs(host_f64(fp8_win["swiglu"])[WIN_ROWS] - oracle.swiglu(a64, c64)) <= Tz)


@pytest.mark.parametrize("cut", [[64] * 7 + [2], [17, 300, 133]])
def test_fp8_window_cuts_and_rows(fp8_win, cut):
    for pb, ref in ((None, "plain"), (fp8_win["pb"], "swiglu")):
        z = q4.qmm_cut_fp8b(fp8_win["pa"], pb, 1024, 2112, fp8_win["xd"], cut)
        torch.cuda.synchronize()
        assert np.array_equal(bits32(z), bits32(fp8_win[ref])), ref
    ref = bits32(fp8_win["swiglu"])
    for r in WIN_ROWS[:5]:
        z1 = q4.qmm_window_fp8b(fp8_win["pa"], fp8_win["pb"], 1024, 2112, fp8_win["xd"][r : r + 1])
        assert np.array_equal(bits32(z1)[0], ref[r]), r
