"""Seeded sweep over shapes, strides and formats the fixed-workload tests do
not reach: K and N at odd multiples of 64, padded row strides on both sides,
float32 and bf16 outputs, the SwiGLU and plain prompt windows, and every
code format (4-, 6-, 8-bit MLX and block FP8).

Every case checks the stated tolerance against the float64 oracle and a bit
rule: a decode row equals its one-row call; a window row equals the same row
computed inside a different cut of the prompt."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import oracle
import synthetic
from tests.gpu_helpers import DEV, bits16, bits32, dev_bf16, dev_f32, dev_weight, host_f64, say
from tests.tolerance import tol, tol_bf16_out, tol_swiglu

pytestmark = pytest.mark.gpu

FORMATS = (4, 6, 8, "fp8")


def _draw_case(seed, decode):
    rng = np.random.default_rng(seed)
    fmt = FORMATS[seed % len(FORMATS)]
    N = 64 * int(rng.integers(1, 7))
    K = 64 * int(rng.choice([1, 3, 5, 9, 17, 33] if decode else [1, 3, 5, 9, 17]))
    if fmt == "fp8":
        N = 128 * int(rng.integers(1, 4))  # whole FP8 scale blocks along N
    rows = int(rng.integers(1, 17)) if decode else int(rng.integers(1, 300))
    pad_x = 8 * int(rng.integers(0, 5))  # bf16 elements: 16-byte multiples
    pad_y = 8 * int(rng.integers(0, 5))  # 16-byte multiples for bf16 and float32 outputs
    return rng, fmt, N, K, rows, pad_x, pad_y


def _weight(rng, fmt, name, N, K):
    if fmt == "fp8":
        w = synthetic.draw_fp8_weight(rng, name, N, K)
        p = q4.pack_fp8b(torch.from_numpy(np.ascontiguousarray(w.w8)).to(DEV), torch.from_numpy(np.ascontiguousarray(w.scales)).to(DEV))
        return w, p
    w = synthetic.draw_qweight(rng, name, N, K, bits=fmt)
    return w, dev_weight(w)


def _oracle(w, fmt, xs):
    if fmt == "fp8":
        return oracle.matmul_rows_fp8(w.w8, w.scales, xs), oracle.error_weight_fp8(w.w8, w.scales, xs)
    return (oracle.matmul_rows(w.wq, w.scales, w.biases, xs, bits=fmt),
            oracle.error_weight(w.wq, w.scales, w.biases, xs, bits=fmt))


def _tol_fmt(fmt):
    return "fp8" if fmt == "fp8" else "affine"


def _padded_bf16(x_bits, pad):
    M, K = x_bits.shape
    buf = torch.zeros((M, K + pad), dtype=torch.bfloat16, device=DEV)
    buf[:, :K] = dev_bf16(x_bits)
    return buf[:, :K]


def _padded_f32(x, pad):
    M, K = x.shape
    buf = torch.zeros((M, K + pad), dtype=torch.float32, device=DEV)
    buf[:, :K] = dev_f32(x)
    return buf[:, :K]


def _out(M, N, pad, dtype):
    return torch.full((M, N + pad), float("nan"), dtype=dtype, device=DEV)[:, :N]


def _qmv(p, fmt, N, K, x, y):
    if fmt == "fp8":
        return q4.qmv_rows_fp8b(p, N, K, x, y=y)
    return q4.qmv_rows(p, N, K, x, y=y, bits=fmt)


def _window(pa, pb, fmt, N, K, x, y):
    if fmt == "fp8":
        return q4.qmm_window_fp8b(pa, pb, N, K, x, y=y)
    return q4.qmm_window(pa, pb, N, K, x, y=y, bits=fmt)


@pytest.mark.parametrize("seed", range(24))
def test_decode_sweep(seed):
    rng, fmt, N, K, R, pad_x, pad_y = _draw_case(seed, decode=True)
    xf32 = bool(seed % 3 == 2)
    say(f"decode sweep seed={seed} fmt={fmt} N={N} K={K} R={R} x={'f32' if xf32 else 'bf16'} pad_x={pad_x} pad_y={pad_y}")
    w, p = _weight(rng, fmt, "w", N, K)
    if xf32:
        x = synthetic.draw_f32_rows(rng, R, K, sigma=0.5)
        xd = _padded_f32(x, pad_x)
        xs = x.astype(np.float64)
    else:
        x = synthetic.draw_bf16_rows(rng, R, K)
        xd = _padded_bf16(x, pad_x)
        xs = x
    y = _out(R, N, pad_y, torch.float32)
    _qmv(p, fmt, N, K, xd, y)
    torch.cuda.synchronize()
    y64, A = _oracle(w, fmt, xs)
    T = tol(A, K, "f32" if xf32 else "bf16", order="decode", fmt=_tol_fmt(fmt))
    got = host_f64(y)
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - y64) <= T), f"max err/T {float(np.max(np.abs(got - y64) / T))}"
    # every row equals its one-row call
    for r in sorted({0, R // 2, R - 1}):
        y1 = _out(1, N, 0, torch.float32)
        _qmv(p, fmt, N, K, xd[r : r + 1], y1)
        torch.cuda.synchronize()
        assert np.array_equal(bits32(y1)[0], bits32(y)[r])


@pytest.mark.parametrize("seed", range(24))
def test_window_sweep(seed):
    rng, fmt, N, K, M, pad_x, pad_y = _draw_case(100 + seed, decode=False)
    swiglu = bool(seed % 2)
    out_dtype = torch.bfloat16 if seed % 3 == 0 else torch.float32
    say(f"window sweep seed={seed} fmt={fmt} N={N} K={K} M={M} swiglu={swiglu} out={out_dtype} pad_x={pad_x} pad_y={pad_y}")
    wa, pa = _weight(rng, fmt, "wa", N, K)
    wb, pb = _weight(rng, fmt, "wb", N, K) if swiglu else (None, None)
    x = synthetic.draw_bf16_rows(rng, M, K)
    xd = _padded_bf16(x, pad_x)
    y = _out(M, N, pad_y, out_dtype)
    _window(pa, pb, fmt, N, K, xd, y)
    torch.cuda.synchronize()
    a64, Aa = _oracle(wa, fmt, x)
    Ta = tol(Aa, K, order="window", fmt=_tol_fmt(fmt))
    if swiglu:
        c64, Ac = _oracle(wb, fmt, x)
        ref, bound = oracle.swiglu(a64, c64), tol_swiglu(a64, c64, Ta, tol(Ac, K, order="window", fmt=_tol_fmt(fmt)))
    else:
        ref, bound = a64, Ta
    if out_dtype == torch.bfloat16:
        got = oracle.bf16_to_f64(bits16(y).view(np.uint16))
        bound = tol_bf16_out(ref, bound)
    else:
        got = host_f64(y)
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= bound), f"max err/bound {float(np.max(np.abs(got - ref) / bound))}"
    # the same rows through a different cut: a window of the first rows, then the rest in two windows
    cut = sorted({int(c) for c in rng.integers(1, M, 2)}) if M > 2 else []
    edges = [0] + cut + [M]
    y2 = _out(M, N, 0, out_dtype)
    for lo, hi in zip(edges[:-1], edges[1:]):
        _window(pa, pb, fmt, N, K, xd[lo:hi], y2[lo:hi])
    torch.cuda.synchronize()
    conv = bits16 if out_dtype == torch.bfloat16 else bits32
    assert np.array_equal(conv(y2), conv(y))
