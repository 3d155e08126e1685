"""Prefill window GEMM on the GPU: float64 parity on the 1000-row prompt and
bit-identity across every cut (64, 128, 256, ragged, single rows)."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import oracle
import synthetic
from tests.gpu_helpers import DEV, bits16, bits32, check_within, dev_bf16, dev_weight, host_f64, say
from tests.tolerance import tol, tol_bf16_out, tol_swiglu

pytestmark = pytest.mark.gpu

# rows at and around every window boundary of the four cuts
SAMPLE_ROWS = [0, 1, 15, 16, 17, 63, 64, 127, 128, 255, 256, 316, 317, 511, 512, 767, 768, 959, 960, 999]


@pytest.fixture(scope="module")
def c3():
    d = synthetic.config(3)
    d["p1"] = dev_weight(d["w1"])
    d["p3"] = dev_weight(d["w3"])
    d["xd"] = dev_bf16(d["x"])
    return d


@pytest.fixture(scope="module")
def c3_whole(c3):
    w1 = c3["w1"]
    z = q4.qmm_window(c3["p1"], c3["p3"], w1.N, w1.K, c3["xd"])
    torch.cuda.synchronize()
    return z


def test_c3_swiglu_parity(c3, c3_whole):
    w1, w3 = c3["w1"], c3["w3"]
    say("c3 pgemm SwiGLU 1000x8192 parity on boundary rows")
    xs = c3["x"][SAMPLE_ROWS]
    a64 = oracle.matmul_rows(w1.wq, w1.scales, w1.biases, xs)
    c64 = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, xs)
    Tz = tol_swiglu(a64, c64, tol(oracle.error_weight(w1.wq, w1.scales, w1.biases, xs), w1.K, order="window"),
                    tol(oracle.error_weight(w3.wq, w3.scales, w3.biases, xs), w3.K, order="window"))
    z = host_f64(c3_whole)[SAMPLE_ROWS]
    ratio = float(np.max(np.abs(z - oracle.swiglu(a64, c64)) / Tz))
    say(f"c3 max err/Tz {ratio:.3g}")
    assert ratio <= 1.0


@pytest.mark.parametrize("cut", ["w64", "w128", "w256", "ragged"])
def test_c3_cuts_bit_identical(c3, c3_whole, cut):
    w1 = c3["w1"]
    say(f"c3 cut {cut}")
    z = q4.qmm_cut(c3["p1"], c3["p3"], w1.N, w1.K, c3["xd"], c3["cuts"][cut])
    torch.cuda.synchronize()
    assert np.array_equal(bits32(z), bits32(c3_whole))


def test_c3_single_row_windows(c3, c3_whole):
    """Every row alone equals the row inside a window (sampled rows)."""
    w1 = c3["w1"]
    say("c3 M=1 windows")
    ref = bits32(c3_whole)
    for r in SAMPLE_ROWS:
        z1 = q4.qmm_window(c3["p1"], c3["p3"], w1.N, w1.K, c3["xd"][r : r + 1])
        assert np.array_equal(bits32(z1)[0], ref[r]), r


def test_c3_bf16_output_is_rne_of_float32(c3, c3_whole):
    w1, w3 = c3["w1"], c3["w3"]
    zb = q4.qmm_window(c3["p1"], c3["p3"], w1.N, w1.K, c3["xd"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    f = c3_whole.cpu().numpy()
    expect = synthetic.bf16_bits_from_f64(f.astype(np.float64))  # f32 -> bf16 RNE
    assert np.array_equal(bits16(zb).view(np.uint16), expect)
    # and against the oracle with the bf16 half-ulp added
    xs = c3["x"][SAMPLE_ROWS[:6]]
    a64 = oracle.matmul_rows(w1.wq, w1.scales, w1.biases, xs)
    c64 = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, xs)
    z64 = oracle.swiglu(a64, c64)
    Tz = tol_swiglu(a64, c64, tol(oracle.error_weight(w1.wq, w1.scales, w1.biases, xs), w1.K, order="window"),
                    tol(oracle.error_weight(w3.wq, w3.scales, w3.biases, xs), w3.K, order="window"))
    zb64 = oracle.bf16_to_f64(bits16(zb).view(np.uint16)[SAMPLE_ROWS[:6]])
    assert np.all(np.abs(zb64 - z64) <= tol_bf16_out(z64, Tz))


@pytest.mark.parametrize("M", [1, 2, 17, 64, 65, 100])
def test_plain_window_parity_and_row_permutation(M):
    d = synthetic.config(2)
    w = synthetic.concat_rows(d["wq"], d["wk"], d["wv"])
    rng = np.random.default_rng(M)
    x = synthetic.draw_bf16_rows(rng, M, w.K)
    say(f"plain pgemm qkv M={M}")
    pk = dev_weight(w)
    xd = dev_bf16(x)
    y = q4.qmm_window(pk, None, w.N, w.K, xd)
    torch.cuda.synchronize()
    check_within(host_f64(y), w, x, label=f"pgemm plain M={M}", order="window")
    perm = rng.permutation(M)
    yp = q4.qmm_window(pk, None, w.N, w.K, xd[torch.from_numpy(perm).to(DEV)])
    assert np.array_equal(bits32(yp), bits32(y)[perm])
    yb = q4.qmm_window(pk, None, w.N, w.K, xd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(bits16(yb).view(np.uint16), synthetic.bf16_bits_from_f64(y.cpu().numpy().astype(np.float64)))


@pytest.mark.parametrize("N,K,M", [(64, 64, 5), (64, 192, 33), (320, 640, 40)])
def test_pgemm_edge_shapes(N, K, M):
    say(f"edge pgemm N={N} K={K} M={M}")
    rng = np.random.default_rng(N * K + M)
    w = synthetic.draw_qweight(rng, "e", N, K)
    w3 = synthetic.draw_qweight(rng, "e3", N, K)
    s = (w.scales.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w.scales = synthetic.bf16_bits_from_f64(s * rng.choice([-1.0, 1.0, 0.0], size=s.shape))
    x = synthetic.bf16_bits_from_f64(rng.normal(0, 1, (M, K)) * rng.choice([1e-4, 1.0, 50.0], (M, K)))
    pk, pk3, xd = dev_weight(w), dev_weight(w3), dev_bf16(x)
    y = host_f64(q4.qmm_window(pk, None, N, K, xd))
    check_within(y, w, x, label="edge pgemm", order="window")
    z = host_f64(q4.qmm_window(pk, pk3, N, K, xd))
    a64 = oracle.matmul_rows(w.wq, w.scales, w.biases, x)
    c64 = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, x)
    Tz = tol_swiglu(a64, c64, tol(oracle.error_weight(w.wq, w.scales, w.biases, x), K, order="window"),
                    tol(oracle.error_weight(w3.wq, w3.scales, w3.biases, x), K, order="window"))
    assert np.all(np.abs(z - oracle.swiglu(a64, c64)) <= Tz)


def test_window_and_decode_orders_differ(c3):
    """Control for the bit tests: the prompt GEMM and the decode matvec use
    different (each fixed) summation orders, and the bit comparisons can see
    that difference on real data."""
    w1 = c3["w1"]
    xs = c3["xd"][:16]
    a_win = bits32(q4.qmm_window(c3["p1"], None, w1.N, w1.K, xs))
    a_dec = bits32(q4.qmv_rows(c3["p1"], w1.N, w1.K, xs))
    assert not np.array_equal(a_win, a_dec)


@pytest.mark.parametrize("rows", [384, 385])
def test_c3_windows_at_the_short_window_boundary(c3, c3_whole, rows):
    """w1/w3 8192 x 2048 with the SwiGLU epilogue: a 384-row window is the
    last one computed on the 64-column workgroups of short windows (3 row
    blocks x 64 column blocks of 128 x 256 would be 192 < 256 workgroups),
    385 rows the first on the 128 x 256 workgroups. Either way every row is
    bit-identical to the same row of the whole 1000-row prompt. The plain
    (no SwiGLU) window of w1 runs on the short-window workgroups at both
    sizes (at most 4 x 32 wide workgroups) and the whole prompt on the wide
    ones (8 x 32): its rows agree too."""
    w1 = c3["w1"]
    say(f"c3 window of {rows} rows at the short-window boundary")
    z = q4.qmm_window(c3["p1"], c3["p3"], w1.N, w1.K, c3["xd"][:rows])
    a = q4.qmm_window(c3["p1"], None, w1.N, w1.K, c3["xd"][:rows])
    a_whole = q4.qmm_window(c3["p1"], None, w1.N, w1.K, c3["xd"])
    torch.cuda.synchronize()
    assert np.array_equal(bits32(z), bits32(c3_whole)[:rows])
    assert np.array_equal(bits32(a), bits32(a_whole)[:rows])


@pytest.mark.parametrize("swiglu", [False, True])
def test_wide_kernel_odd_groups_and_partial_column_block(swiglu):
    """4-bit windows large enough for the 128 x 256 (SwiGLU: 128 x 128)
    workgroups, with an odd group count (K = 64 * 9: the pipeline's last
    group pair is half empty) and a last column block partly past N
    (N = 16 * 256 + 64). Sampled rows, including the last row block and all
    N columns, are within the window bound of the oracle; a 100-row window
    (on the short-window workgroups) and single rows are bit-identical to the
    same rows of the wide launch."""
    N, K = 4160, 576
    M = 1000 if swiglu else 2000
    cols = 128 if swiglu else 256
    assert -(-N // cols) * -(-M // 128) >= 256 and -(-N // cols) < 256  # wide, then short-window workgroups
    say(f"wide pgemm N={N} K={K} M={M} swiglu={swiglu}")
    rng = np.random.default_rng(4160 + swiglu)
    w = synthetic.draw_qweight(rng, "wa", N, K)
    w3 = synthetic.draw_qweight(rng, "wb", N, K)
    x = synthetic.draw_bf16_rows(rng, M, K)
    pk, pk3, xd = dev_weight(w), dev_weight(w3), dev_bf16(x)
    pb = pk3 if swiglu else None
    y = q4.qmm_window(pk, pb, N, K, xd)
    y100 = q4.qmm_window(pk, pb, N, K, xd[:100])
    torch.cuda.synchronize()
    rows = [0, 1, 99, 100, 127, 128, 500, M - 129, M - 128, M - 2, M - 1]
    xs = x[rows]
    if swiglu:
        a64 = oracle.matmul_rows(w.wq, w.scales, w.biases, xs)
        c64 = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, xs)
        Tz = tol_swiglu(a64, c64, tol(oracle.error_weight(w.wq, w.scales, w.biases, xs), K, order="window"),
                        tol(oracle.error_weight(w3.wq, w3.scales, w3.biases, xs), K, order="window"))
        ratio = float(np.max(np.abs(host_f64(y)[rows] - oracle.swiglu(a64, c64)) / Tz))
        assert ratio <= 1.0, ratio
    else:
        check_within(host_f64(y)[rows], w, x, rows=rows, label="wide pgemm", order="window")
    ref = bits32(y)
    assert np.array_equal(bits32(y100), ref[:100])
    for r in (0, 99, M - 1):
        y1 = q4.qmm_window(pk, pb, N, K, xd[r : r + 1])
        assert np.array_equal(bits32(y1)[0], ref[r]), r


@pytest.mark.parametrize("layout", ["ldy_not_multiple_of_8", "rows_not_16_byte_aligned"])
def test_wide_swiglu_bf16_output_rows_of_any_alignment(c3, c3_whole, layout):
    """The 1000-row w1/w3 window (512 wide workgroups) writing bf16 into rows
    that a 16-byte store cannot reach: row stride N + 4, or the output
    starting one element into each row. Values equal the round-to-nearest-even
    bf16 of the float32 result, and the padding around the rows is untouched."""
    w1 = c3["w1"]
    N, K, M = w1.N, w1.K, c3["x"].shape[0]
    say(f"c3 pgemm SwiGLU bf16 out, {layout}")
    nan = float("nan")
    if layout == "ldy_not_multiple_of_8":
        big = torch.full((M, N + 4), nan, dtype=torch.bfloat16, device=DEV)
        y, c0 = big[:, :N], 0
    else:
        big = torch.full((M, N + 8), nan, dtype=torch.bfloat16, device=DEV)
        y, c0 = big[:, 1 : N + 1], 1
    q4.qmm_window(c3["p1"], c3["p3"], N, K, c3["xd"], y=y)
    torch.cuda.synchronize()
    expect = synthetic.bf16_bits_from_f64(c3_whole.cpu().numpy().astype(np.float64))
    got = bits16(big).view(np.uint16)
    assert np.array_equal(got[:, c0 : c0 + N], expect)
    pad = np.delete(got, np.arange(c0, c0 + N), axis=1)
    assert np.all((pad & 0x7FFF) > 0x7F80)  # still NaN


@pytest.mark.parametrize("swiglu,out_bf16", [(False, False), (False, True), (True, False), (True, True)])
def test_short_windows_match_the_whole_prompt(swiglu, out_bf16):
    """Short windows (one to a few hundred rows) of a wide-K weight run on the
    workgroups of short windows (one 32 x 32 tile each, products of several
    groups at once, folded in order), the whole prompt on the 128 x 256
    (SwiGLU 128 x 128) workgroups: every row's bits agree, for w2's shape
    (2048 x 8192) and an odd group count (K = 64 * 63)."""
    K = 8192 if not swiglu else 4032
    N = 2048
    M = 4096 if not swiglu else 2048  # enough rows for the wide workgroups
    say(f"short windows vs whole prompt N={N} K={K} swiglu={swiglu} bf16={out_bf16}")
    rng = np.random.default_rng(N + K + swiglu)
    w = synthetic.draw_qweight(rng, "a", N, K)
    w3 = synthetic.draw_qweight(rng, "b", N, K)
    pk, pk3 = dev_weight(w), dev_weight(w3)
    pb = pk3 if swiglu else None
    x = synthetic.draw_bf16_rows(rng, M, K)
    xd = dev_bf16(x)
    dt = torch.bfloat16 if out_bf16 else torch.float32
    whole = q4.qmm_window(pk, pb, N, K, xd, out_dtype=dt)
    torch.cuda.synchronize()
    ref = bits16(whole) if out_bf16 else bits32(whole)
    for r0, rows in ((0, 128), (1000, 128), (4000 % M, 96), (77, 1), (300, 17), (M - 33, 33)):
        y = q4.qmm_window(pk, pb, N, K, xd[r0 : r0 + rows], out_dtype=dt)
        torch.cuda.synchronize()
        got = bits16(y) if out_bf16 else bits32(y)
        assert np.array_equal(got, ref[r0 : r0 + rows]), (r0, rows)
    # and one window's rows against the oracle
    rows = [0, 63, 127]
    if swiglu:
        a64 = oracle.matmul_rows(w.wq, w.scales, w.biases, x[rows])
        c64 = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, x[rows])
        Tz = tol_swiglu(a64, c64, tol(oracle.error_weight(w.wq, w.scales, w.biases, x[rows]), K, order="window"),
                        tol(oracle.error_weight(w3.wq, w3.scales, w3.biases, x[rows]), K, order="window"))
        z64 = oracle.swiglu(a64, c64)
        got64 = host_f64(q4.qmm_window(pk, pb, N, K, xd[:128]))[rows]
        assert np.all(np.abs(got64 - z64) <= Tz)
    else:
        check_within(host_f64(q4.qmm_window(pk, None, N, K, xd[:128]))[rows], w, x, rows=rows, label="short window w2", order="window")


@pytest.mark.parametrize("swiglu,out_bf16", [(False, False), (True, False), (True, True)])
def test_two_round_short_windows_match_the_whole_prompt(swiglu, out_bf16):
    """Windows whose 32 x 32 tiles number between one and two per compute unit
    (N = 4096: 128 rows are 512 tiles, 65 and 96 rows 384) run with two
    short-window workgroups sharing a compute unit (SwiGLU: the 2-producer
    form); every row's bits equal the whole prompt's on the wide workgroups."""
    N = 4096
    K = 8192 if not swiglu else 4032
    M = 2048
    say(f"two-round short windows vs whole prompt N={N} K={K} swiglu={swiglu} bf16={out_bf16}")
    rng = np.random.default_rng(N + K + 7 * swiglu)
    w = synthetic.draw_qweight(rng, "a", N, K)
    pk = dev_weight(w)
    pb = dev_weight(synthetic.draw_qweight(rng, "b", N, K)) if swiglu else None
    xd = dev_bf16(synthetic.draw_bf16_rows(rng, M, K))
    dt = torch.bfloat16 if out_bf16 else torch.float32
    bits = bits16 if out_bf16 else bits32
    ref = bits(q4.qmm_window(pk, pb, N, K, xd, out_dtype=dt))
    for r0, rows in ((0, 128), (1000, 96), (300, 65), (M - 33, 33), (5, 1)):
        y = q4.qmm_window(pk, pb, N, K, xd[r0 : r0 + rows], out_dtype=dt)
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), ref[r0 : r0 + rows]), (r0, rows)


@pytest.mark.parametrize("N,K,M,swiglu", [(64, 64, 1, False), (64, 128, 31, True), (128, 64, 32, False), (128, 192, 33, True),
                                          (192, 320, 63, False), (256, 64 * 17, 64, True), (1024, 576, 65, False)])
def test_short_window_edge_shapes_against_single_rows_and_oracle(N, K, M, swiglu):
    """Windows on the short-window workgroups at the edges of their 32-row
    blocks (31, 32, 33, 63, 64, 65 rows), with one, two, odd and chunk-crossing
    group counts (K = 64 .. 64 * 17), plain and SwiGLU: within the window bound
    of the oracle, and every row bit-identical to that row alone (also a
    short-window launch) and in bf16 to the RNE of the float32 result."""
    say(f"short window N={N} K={K} M={M} swiglu={swiglu}")
    rng = np.random.default_rng(N * 7 + K + M)
    w = synthetic.draw_qweight(rng, "a", N, K)
    w3 = synthetic.draw_qweight(rng, "b", N, K)
    pk, pk3 = dev_weight(w), dev_weight(w3)
    pb = pk3 if swiglu else None
    x = synthetic.draw_bf16_rows(rng, M, K)
    xd = dev_bf16(x)
    y = q4.qmm_window(pk, pb, N, K, xd)
    yb = q4.qmm_window(pk, pb, N, K, xd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = bits32(y)
    for r in sorted({0, M // 2, M - 1}):
        y1 = q4.qmm_window(pk, pb, N, K, xd[r : r + 1])
        assert np.array_equal(bits32(y1)[0], ref[r]), r
    assert np.array_equal(bits16(yb).view(np.uint16), synthetic.bf16_bits_from_f64(y.cpu().numpy().astype(np.float64)))
    if swiglu:
        a64 = oracle.matmul_rows(w.wq, w.scales, w.biases, x)
        c64 = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, x)
        Tz = tol_swiglu(a64, c64, tol(oracle.error_weight(w.wq, w.scales, w.biases, x), K, order="window"),
                        tol(oracle.error_weight(w3.wq, w3.scales, w3.biases, x), K, order="window"))
        assert np.all(np.abs(host_f64(y) - oracle.swiglu(a64, c64)) <= Tz)
    else:
        check_within(host_f64(y), w, x, label="short window edge", order="window")
