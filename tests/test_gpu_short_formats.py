"""Short windows of 6-bit, 8-bit and block-FP8 weights against the whole
prompt on the wide 128 x 256 workgroups: every row's bits agree (TensorFold
PR #1696, later revision, "Checks": a row alone equals the row inside a
window; PR #1514, "What changes": the 4-, 6- and 8-bit checkpoints served as
stored; PR #1696, "Checks": block FP8 weights served weight-only). The whole
prompt (8192 rows) is large enough for the wide kernel. The windows (1 to
1536 rows) run on the two short-window kernels: on the dataflow workgroups
(one 32 x 32 tile each, products of several groups at once, folded in order)
in one round, in the two-workgroups-per-CU SwiGLU form and in up to four
rounds of plain tiles; past that (1024- and 1536-row SwiGLU windows, the
1536-row plain window) on the 64-column narrow workgroups. One window per
case is also checked against the float64 oracle."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import oracle
import synthetic
from tests.gpu_helpers import DEV, bits16, bits32, check_within, dev_bf16, dev_weight, host_f64, say
from tests.tolerance import tol, tol_swiglu

pytestmark = pytest.mark.gpu

N, K, M = 1024, 64 * 33, 8192  # an odd group count
# 1 to 448 rows: one or two rounds; 1024 and 1536 rows: up to 4 (SwiGLU) and 6 (plain) tiles per CU
WINDOWS = ((0, 128), (1000, 96), (300, 65), (M - 33, 33), (5, 1), (2000, 448), (4096, 1024), (5200, 1536))


def _pack(fmt, w):
    if fmt == "fp8":
        return q4.pack_fp8b(torch.from_numpy(np.ascontiguousarray(w.w8)).to(DEV), torch.from_numpy(np.ascontiguousarray(w.scales)).to(DEV))
    return dev_weight(w)


def _window(fmt, pa, pb, xd, dt):
    if fmt == "fp8":
        return q4.qmm_window_fp8b(pa, pb, N, K, xd, out_dtype=dt)
    return q4.qmm_window(pa, pb, N, K, xd, bits=fmt, out_dtype=dt)


@pytest.fixture(scope="module", params=[6, 8, "fp8"])
def fmt_case(request):
    fmt = request.param
    rng = np.random.default_rng(901 if fmt == "fp8" else 900 + fmt)
    if fmt == "fp8":
        a, b = synthetic.draw_fp8_weight(rng, "a", N, K), synthetic.draw_fp8_weight(rng, "b", N, K)
    else:
        a, b = synthetic.draw_qweight(rng, "a", N, K, bits=fmt), synthetic.draw_qweight(rng, "b", N, K, bits=fmt)
    x = synthetic.draw_bf16_rows(rng, M, K)
    return {"fmt": fmt, "a": a, "b": b, "x": x, "pa": _pack(fmt, a), "pb": _pack(fmt, b), "xd": dev_bf16(x)}


@pytest.mark.parametrize("swiglu,out_bf16", [(False, False), (True, False), (True, True)])
def test_short_windows_of_wider_codes_match_the_whole_prompt(fmt_case, swiglu, out_bf16):
    fmt = fmt_case["fmt"]
    say(f"short windows fmt={fmt} swiglu={swiglu} bf16={out_bf16} vs the whole prompt")
    pb = fmt_case["pb"] if swiglu else None
    dt = torch.bfloat16 if out_bf16 else torch.float32
    bits = bits16 if out_bf16 else bits32
    ref = bits(_window(fmt, fmt_case["pa"], pb, fmt_case["xd"], dt))
    torch.cuda.synchronize()
    for r0, rows in WINDOWS:
        y = _window(fmt, fmt_case["pa"], pb, fmt_case["xd"][r0 : r0 + rows], dt)
        torch.cuda.synchronize()
        assert np.array_equal(bits(y), ref[r0 : r0 + rows]), (r0, rows)


@pytest.mark.parametrize("r0,nrows,rows", [(0, 96, [0, 37, 95]), (4096, 1024, [0, 513, 1023])])
def test_short_window_of_wider_codes_within_oracle_bound(fmt_case, r0, nrows, rows):
    """96 rows: dataflow workgroups for both products; 1024 rows: dataflow
    workgroups for the plain product, narrow workgroups for SwiGLU."""
    fmt = fmt_case["fmt"]
    say(f"short window fmt={fmt} rows {r0}+{nrows} against the oracle")
    xw = fmt_case["x"][r0 : r0 + nrows]
    xs = xw[rows]
    a, b = fmt_case["a"], fmt_case["b"]
    xd = fmt_case["xd"][r0 : r0 + nrows]
    y = host_f64(_window(fmt, fmt_case["pa"], None, xd, torch.float32))[rows]
    z = host_f64(_window(fmt, fmt_case["pa"], fmt_case["pb"], xd, torch.float32))[rows]
    if fmt == "fp8":
        a64 = oracle.matmul_rows_fp8(a.w8, a.scales, xs)
        c64 = oracle.matmul_rows_fp8(b.w8, b.scales, xs)
        Ta = tol(oracle.error_weight_fp8(a.w8, a.scales, xs), K, order="window", fmt="fp8")
        Tc = tol(oracle.error_weight_fp8(b.w8, b.scales, xs), K, order="window", fmt="fp8")
        assert np.all(np.abs(y - a64) <= Ta)
    else:
        check_within(y, a, xw, rows=rows, label=f"short window {fmt}-bit", order="window")
        a64 = oracle.matmul_rows(a.wq, a.scales, a.biases, xs, bits=fmt)
        c64 = oracle.matmul_rows(b.wq, b.scales, b.biases, xs, bits=fmt)
        Ta = tol(oracle.error_weight(a.wq, a.scales, a.biases, xs, bits=fmt), K, order="window")
        Tc = tol(oracle.error_weight(b.wq, b.scales, b.biases, xs, bits=fmt), K, order="window")
    assert np.all(np.abs(z - oracle.swiglu(a64, c64)) <= tol_swiglu(a64, c64, Ta, Tc))


@pytest.mark.parametrize("fmt", [6, 8, "fp8"])
def test_narrow_workgroups_odd_shape(fmt):
    """N = 1088 (17 narrow workgroups of 64 columns, 34 of 32 for SwiGLU; the
    wide workgroups' last column block is partly past N) and K = 64 * 9 (the
    last group pair half empty), on windows of 1024 and 2048 rows that take
    the narrow workgroups. Their rows equal the whole prompt's (8192 rows,
    wide workgroups) bit for bit, and sampled rows are within the window
    bound of the float64 oracle."""
    N2, K2, M2 = 1088, 64 * 9, 8192
    say(f"narrow workgroups fmt={fmt} N={N2} K={K2}")
    rng = np.random.default_rng(1088 + (9 if fmt == "fp8" else fmt))
    if fmt == "fp8":
        a, b = synthetic.draw_fp8_weight(rng, "a", N2, K2), synthetic.draw_fp8_weight(rng, "b", N2, K2)
    else:
        a, b = synthetic.draw_qweight(rng, "a", N2, K2, bits=fmt), synthetic.draw_qweight(rng, "b", N2, K2, bits=fmt)
    pa, pb = _pack(fmt, a), _pack(fmt, b)
    x = synthetic.draw_bf16_rows(rng, M2, K2)
    xd = dev_bf16(x)

    def win(p_b, xs):
        if fmt == "fp8":
            return q4.qmm_window_fp8b(pa, p_b, N2, K2, xs, out_dtype=torch.float32)
        return q4.qmm_window(pa, p_b, N2, K2, xs, bits=fmt, out_dtype=torch.float32)

    for p_b, r0, rows in ((None, 1000, 2048), (pb, 3000, 1024)):
        ref = bits32(win(p_b, xd))
        y = win(p_b, xd[r0 : r0 + rows])
        torch.cuda.synchronize()
        assert np.array_equal(bits32(y), ref[r0 : r0 + rows]), (p_b is None, r0, rows)
    sample = [0, 511, 1023]
    xs = x[3000:4024][sample]
    z = host_f64(win(pb, xd[3000:4024]))[sample]
    if fmt == "fp8":
        a64, c64 = oracle.matmul_rows_fp8(a.w8, a.scales, xs), oracle.matmul_rows_fp8(b.w8, b.scales, xs)
        Ta = tol(oracle.error_weight_fp8(a.w8, a.scales, xs), K2, order="window", fmt="fp8")
        Tc = tol(oracle.error_weight_fp8(b.w8, b.scales, xs), K2, order="window", fmt="fp8")
    else:
        a64 = oracle.matmul_rows(a.wq, a.scales, a.biases, xs, bits=fmt)
        c64 = oracle.matmul_rows(b.wq, b.scales, b.biases, xs, bits=fmt)
        Ta = tol(oracle.error_weight(a.wq, a.scales, a.biases, xs, bits=fmt), K2, order="window")
        Tc = tol(oracle.error_weight(b.wq, b.scales, b.biases, xs, bits=fmt), K2, order="window")
    assert np.all(np.abs(z - oracle.swiglu(a64, c64)) <= tol_swiglu(a64, c64, Ta, Tc))


@pytest.mark.parametrize("fmt", [4, 6, 8, "fp8"])
@pytest.mark.parametrize("groups", [1, 2, 9])
def test_narrow_workgroups_group_counts(fmt, groups):
    """K of one, two and nine groups on windows that take the 64-column narrow
    workgroups: 128 and 100 rows of w1/w3 + SwiGLU with N = 8192 and of a
    plain weight with N = 16384 (more 32 x 32 tiles than the dataflow kernel
    takes, fewer than 256 wide workgroups). The narrow kernel folds each
    group's products during the next group and the last group's after its
    loop; every row must equal the row of a 512-row prompt on the wide
    workgroups, which fold at once, bit for bit."""
    K2, M2 = 64 * groups, 512
    say(f"narrow group counts fmt={fmt} K={K2}")
    rng = np.random.default_rng(7000 + 10 * groups + (9 if fmt == "fp8" else fmt))

    def draw(name, n):
        if fmt == "fp8":
            return synthetic.draw_fp8_weight(rng, name, n, K2)
        return synthetic.draw_qweight(rng, name, n, K2, bits=fmt)

    xd = dev_bf16(synthetic.draw_bf16_rows(rng, M2, K2))
    for swiglu, N2 in ((True, 8192), (False, 16384)):
        pa = _pack(fmt, draw("a", N2))
        pb = _pack(fmt, draw("b", N2)) if swiglu else None

        def win(xs):
            if fmt == "fp8":
                return q4.qmm_window_fp8b(pa, pb, N2, K2, xs, out_dtype=torch.float32)
            return q4.qmm_window(pa, pb, N2, K2, xs, bits=fmt, out_dtype=torch.float32)

        ref = bits32(win(xd))
        for r0, rows in ((0, 128), (384, 128), (200, 100)):
            y = win(xd[r0 : r0 + rows])
            torch.cuda.synchronize()
            assert np.array_equal(bits32(y), ref[r0 : r0 + rows]), (swiglu, r0, rows)
