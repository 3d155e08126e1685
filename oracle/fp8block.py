"""Plain, slow, float64 oracle for the block-FP8 weight-only matmul.

TEST INFRASTRUCTURE, like the rest of ``oracle/``: only tests, the smoke
check and the benchmark's CPU baseline use it; it shares no code with the
HIP kernels or their binding.

What it computes (TensorFold PR #1696, first revision, "Stacked on" and
"Checks": the CUDA engine this backend builds on and is checked against
serves the LFM3 block FP8 export weight-only beside the MLX 4-bit export).
The pages name the format without describing it; the reading here is the
common block-FP8 checkpoint layout:

    w8[n][k]     one OCP FP8 E4M3 byte per weight (sign, 4 exponent bits with
                 bias 7, 3 mantissa bits; exponent field 0 is subnormal,
                 0x7F and 0xFF are NaN, the largest finite value is 448)
    s[i][j]      one float32 scale per 128 x 128 block: rows 128 i .. + 127,
                 columns 128 j .. + 127 (partial blocks at the edges)
    w[n][k]      = e4m3(w8[n][k]) * s[n // 128][k // 128]
    y[m][n]      = sum_k w[n][k] * x[m][k]                   float64

"Weight-only": the activations stay bf16 (or float32); nothing is
requantized.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from .q4g64 import activations_f64

BLOCK = 128


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode OCP FP8 E4M3 bytes to float64, field by field."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def dequantize_fp8(w8, scales, N: int, K: int) -> np.ndarray:
    """Float64 weights w[n][k] = e4m3(w8[n][k]) * s[n // 128][k // 128]."""
    w8 = np.asarray(w8, dtype=np.uint8).reshape(N, K)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    if s.shape != (-(-N // BLOCK), -(-K // BLOCK)):
        raise ValueError("scales must be [ceil(N/128)][ceil(K/128)]")
    rows = np.arange(N) // BLOCK
    cols = np.arange(K) // BLOCK
    return e4m3_to_f64(w8) * s[rows][:, cols]


def matmul_rows_fp8(w8, scales, x, cols=None) -> np.ndarray:
    """y[m][n] = sum_k w[n][k] x[m][k] in float64 (numpy dgemm on the
    dequantized weights). ``cols`` restricts the output columns."""
    X = activations_f64(x)
    K = X.shape[1]
    w8 = np.asarray(w8, dtype=np.uint8)
    N = w8.shape[0]
    W = dequantize_fp8(w8, scales, N, K)
    if cols is not None:
        W = W[np.asarray(cols)]
    return X @ W.T


def error_weight_fp8(w8, scales, x, cols=None) -> np.ndarray:
    """A[m][n] = sum_k |w[n][k]| |x[m][k]|, the scale of every rounding bound."""
    X = np.abs(activations_f64(x))
    K = X.shape[1]
    w8 = np.asarray(w8, dtype=np.uint8)
    W = np.abs(dequantize_fp8(w8, scales, w8.shape[0], K))
    if cols is not None:
        W = W[np.asarray(cols)]
    return X @ W.T


def matmul_rows_fp8_exact(w8, scales, x, cols=None) -> np.ndarray:
    """Correctly rounded float64 y by ``math.fsum`` over the K exact products
    (4 significant bits x 24 x 24 fit in 53)."""
    X = activations_f64(x)
    M, K = X.shape
    w8 = np.asarray(w8, dtype=np.uint8)
    N = w8.shape[0]
    W = dequantize_fp8(w8, scales, N, K)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    y = np.empty((M, len(cols)))
    for i in range(M):
        for j, n in enumerate(cols):
            y[i, j] = math.fsum(W[n] * X[i])
    return y


def _e4m3_fraction(code: int) -> Fraction:
    """One E4M3 byte as an exact rational, from its bit fields."""
    sign = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 64)
    return sign * (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


def matmul_rows_fp8_fraction(w8, scales, x) -> list:
    """Exact rational y by brute force, one weight at a time (tiny shapes)."""
    X = activations_f64(x)
    M, K = X.shape
    w8 = np.asarray(w8, dtype=np.uint8)
    N = w8.shape[0]
    s = np.asarray(scales, dtype=np.float32)
    out = []
    for i in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += _e4m3_fraction(int(w8[n][k])) * Fraction(float(s[n // BLOCK][k // BLOCK])) * Fraction(float(X[i][k]))
            row.append(acc)
        out.append(row)
    return out
