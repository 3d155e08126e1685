"""MLX 6- and 8-bit group-64 weights (PR #1514, "What changes": the 4-, 6-
and 8-bit checkpoints are served as stored) through the same boundary: pack
is bit-exact against the layout model and invertible; the decode matvecs sit
within the stated tolerance of the float64 oracle and keep the N-row = 1-row
bit rule; the fused SwiGLU call equals silu of one call times the other."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import oracle
import synthetic
from tests.gpu_helpers import DEV, bits32, check_within, dev_bf16, dev_f32, dev_weight, host_f64, say
from tests.layout_model import pack_model_bits, packed_bytes_bits
from tests.tolerance import tol, tol_swiglu

pytestmark = pytest.mark.gpu

BITS = [6, 8]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("N,K", [(64, 64), (64, 192), (128, 640), (64, 2048)])
def test_wide_pack_bit_exact_and_invertible(bits, N, K):
    say(f"pack bits={bits} N={N} K={K}")
    rng = np.random.default_rng(1000 * bits + N + K)
    w = synthetic.draw_qweight(rng, "w", N, K, bits=bits)
    w.scales = rng.integers(0, 1 << 16, w.scales.shape, dtype=np.uint16)
    w.biases = rng.integers(0, 1 << 16, w.biases.shape, dtype=np.uint16)
    packed = dev_weight(w)
    torch.cuda.synchronize()
    assert packed.numel() == packed_bytes_bits(N, K, bits) == q4.packed_bytes(N, K, bits)
    model = pack_model_bits(oracle.unpack_codes(w.wq, K, bits), w.scales, w.biases, N, K, bits)
    assert np.array_equal(packed.cpu().numpy(), model)
    wq, sc, bi = q4.unpack(packed, N, K, bits=bits)
    torch.cuda.synchronize()
    assert np.array_equal(wq.cpu().numpy().view(np.uint32), w.wq)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), w.scales)
    assert np.array_equal(bi.cpu().numpy().view(np.uint16), w.biases)


@pytest.fixture(scope="module", params=BITS)
def wide(request):
    bits = request.param
    rng = np.random.default_rng(60 + bits)
    d = {"bits": bits}
    # q/k/v-shaped (3072 x 2048) and w2-shaped (2048 x 8192) matrices
    d["qkv"] = synthetic.draw_qweight(rng, "qkv", 3072, 2048, bits=bits)
    d["w2"] = synthetic.draw_qweight(rng, "w2", 2048, 8192, bits=bits)
    d["w1"] = synthetic.draw_qweight(rng, "w1", 1024, 2048, bits=bits)
    d["w3"] = synthetic.draw_qweight(rng, "w3", 1024, 2048, bits=bits)
    d["x"] = synthetic.draw_bf16_rows(rng, 16, 2048)
    d["xf"] = synthetic.draw_f32_rows(rng, 8, 8192, sigma=0.05)
    for k in ("qkv", "w2", "w1", "w3"):
        d["p_" + k] = dev_weight(d[k])
    return d


@pytest.mark.parametrize("R", [1, 3, 16])
def test_wide_qmv_bf16_within_tolerance(wide, R):
    w = wide["qkv"]
    say(f"qmv_rows bits={wide['bits']} {w.N}x{w.K} R={R}")
    cols = np.arange(0, w.N, 7)
    y = q4.qmv_rows(wide["p_qkv"], w.N, w.K, dev_bf16(wide["x"][:R]), bits=wide["bits"])
    torch.cuda.synchronize()
    check_within(host_f64(y)[:, cols], w, wide["x"][:R], cols=cols, label=f"bits={wide['bits']} R={R}", order="decode")


@pytest.mark.parametrize("R", [1, 5])
def test_wide_qmv_f32_within_tolerance(wide, R):
    w = wide["w2"]
    say(f"qmv_rows f32 x bits={wide['bits']} {w.N}x{w.K} R={R}")
    cols = np.arange(3, w.N, 5)
    y = q4.qmv_rows(wide["p_w2"], w.N, w.K, dev_f32(wide["xf"][:R]), bits=wide["bits"])
    torch.cuda.synchronize()
    check_within(host_f64(y)[:, cols], w, wide["xf"][:R], cols=cols, x_dtype="f32", label=f"bits={wide['bits']} f32 R={R}", order="decode")


def test_wide_rows_bit_equal_to_one_row(wide):
    say(f"qmv_rows bits={wide['bits']} N-row vs 1-row")
    w = wide["qkv"]
    xd = dev_bf16(wide["x"])
    ones = [bits32(q4.qmv_rows(wide["p_qkv"], w.N, w.K, xd[r : r + 1], bits=wide["bits"])) for r in range(16)]
    for R in (2, 5, 16):
        yR = bits32(q4.qmv_rows(wide["p_qkv"], w.N, w.K, xd[:R], bits=wide["bits"]))
        for r in range(R):
            assert np.array_equal(yR[r], ones[r][0]), (R, r)
    w2 = wide["w2"]
    xf = dev_f32(wide["xf"])
    yR = bits32(q4.qmv_rows(wide["p_w2"], w2.N, w2.K, xf, bits=wide["bits"]))
    for r in (0, 7):
        assert np.array_equal(yR[r], bits32(q4.qmv_rows(wide["p_w2"], w2.N, w2.K, xf[r : r + 1], bits=wide["bits"]))[0])


@pytest.mark.parametrize("R", [1, 4])
def test_wide_w13_swiglu(wide, R):
    bits = wide["bits"]
    w1, w3 = wide["w1"], wide["w3"]
    say(f"qmv_w13_swiglu bits={bits} {w1.N}x{w1.K} R={R}")
    xd = dev_bf16(wide["x"][:R])
    z = q4.qmv_w13_swiglu(wide["p_w1"], wide["p_w3"], w1.N, w1.K, xd, bits=bits)
    a = q4.qmv_rows(wide["p_w1"], w1.N, w1.K, xd, bits=bits)
    c = q4.qmv_rows(wide["p_w3"], w3.N, w3.K, xd, bits=bits)
    torch.cuda.synchronize()
    # the two matrices share the fold of qmv_rows: a and c are the same bits
    a64 = oracle.matmul_rows(w1.wq, w1.scales, w1.biases, wide["x"][:R], bits=bits)
    c64 = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, wide["x"][:R], bits=bits)
    Ta = tol(oracle.error_weight(w1.wq, w1.scales, w1.biases, wide["x"][:R], bits=bits), w1.K, order="decode")
    Tc = tol(oracle.error_weight(w3.wq, w3.scales, w3.biases, wide["x"][:R], bits=bits), w3.K, order="decode")
    assert np.all(np.abs(host_f64(a) - a64) <= Ta)
    assert np.all(np.abs(host_f64(c) - c64) <= Tc)
    Tz = tol_swiglu(a64, c64, Ta, Tc)
    assert np.all(np.abs(host_f64(z) - oracle.swiglu(a64, c64)) <= Tz)


# --------------------------------------------------------- prompt windows

WIN_ROWS = [0, 1, 63, 64, 127, 128, 255, 256, 299, 300, 449]


@pytest.fixture(scope="module", params=BITS)
def wide_win(request):
    bits = request.param
    rng = np.random.default_rng(80 + bits)
    d = {"bits": bits}
    # K = 2112 = 33 groups: an odd group count leaves a half-filled last pair
    d["a"] = synthetic.draw_qweight(rng, "a", 1024, 2112, bits=bits)
    d["b"] = synthetic.draw_qweight(rng, "b", 1024, 2112, bits=bits)
    d["x"] = synthetic.draw_bf16_rows(rng, 450, 2112)
    d["pa"], d["pb"], d["xd"] = dev_weight(d["a"]), dev_weight(d["b"]), dev_bf16(d["x"])
    d["plain"] = q4.qmm_window(d["pa"], None, 1024, 2112, d["xd"], bits=bits)
    d["swiglu"] = q4.qmm_window(d["pa"], d["pb"], 1024, 2112, d["xd"], bits=bits)
    torch.cuda.synchronize()
    return d


def test_wide_window_plain_parity(wide_win):
    bits, a = wide_win["bits"], wide_win["a"]
    say(f"qmm_window bits={bits} {a.N}x{a.K} M=450 plain")
    check_within(host_f64(wide_win["plain"])[WIN_ROWS], a, wide_win["x"], rows=WIN_ROWS, label=f"window bits={bits}", order="window")


def test_wide_window_swiglu_parity(wide_win):
    bits, a, b = wide_win["bits"], wide_win["a"], wide_win["b"]
    say(f"qmm_window bits={bits} SwiGLU parity")
    xs = wide_win["x"][WIN_ROWS]
    a64 = oracle.matmul_rows(a.wq, a.scales, a.biases, xs, bits=bits)
    c64 = oracle.matmul_rows(b.wq, b.scales, b.biases, xs, bits=bits)
    Tz = tol_swiglu(a64, c64, tol(oracle.error_weight(a.wq, a.scales, a.biases, xs, bits=bits), a.K, order="window"),
                    tol(oracle.error_weight(b.wq, b.scales, b.biases, xs, bits=bits), b.K, order="window"))
    z = host_f64(wide_win["swiglu"])[WIN_ROWS]
    assert np.all(np.abs(z - oracle.swiglu(a64, c64)) <= Tz)


@pytest.mark.parametrize("cut", [[64] * 7 + [2], [128] * 3 + [66], [17, 300, 133]])
def test_wide_window_cuts_bit_identical(wide_win, cut):
    bits = wide_win["bits"]
    say(f"qmm_cut bits={bits} cut={cut[:3]}...")
    for pb, ref in ((None, "plain"), (wide_win["pb"], "swiglu")):
        z = q4.qmm_cut(wide_win["pa"], pb, 1024, 2112, wide_win["xd"], cut, bits=bits)
        torch.cuda.synchronize()
        assert np.array_equal(bits32(z), bits32(wide_win[ref])), ref


def test_wide_window_single_rows(wide_win):
    bits = wide_win["bits"]
    ref = bits32(wide_win["swiglu"])
    for r in WIN_ROWS:
        z1 = q4.qmm_window(wide_win["pa"], wide_win["pb"], 1024, 2112, wide_win["xd"][r : r + 1], bits=bits)
        assert np.array_equal(bits32(z1)[0], ref[r]), r
