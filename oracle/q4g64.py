"""Plain, slow, float64 oracle for the q4g64 weight-only matmul.

TEST INFRASTRUCTURE. Nothing in the product path may import, call or run this
module; it shares no code with the HIP kernels or their binding. Its only
inputs are the canonical tensors made by ``synthetic`` (or hand-written test
values).

What it computes (TensorFold PR #1696, "What it adds": the LFM3 weights are
MLX 4-bit, group 64, read as stored; later revision, "What it adds" > prompt
GEMM: weight tiles are dequantized as they are loaded and every output is a
dot product over k, summed per 64-wide k block):

    q[n][k] = (wq[n][k // 8] >> (4 * (k % 8))) & 0xF      low nibble first
    w[n][k] = S[n][k // 64] * q[n][k] + B[n][k // 64]      affine dequantization
    y[m][n] = sum_k w[n][k] * x[m][k]                      float64
    z       = silu(a) * c,  silu(a) = a / (1 + exp(-a))    SwiGLU (PR #1696,
                                                           "What it adds": kernels)

Readings where the pages are silent: the dequantization is affine ``s*q + b``
with no zero point subtracted (the MLX convention, with the per-group bias
carrying the offset); codes are packed low nibble first; a group is 64
consecutive k of one output row.

Parity pins (tests/test_oracle_pins.py): hand-worked unpack and dequant words,
one-hot and all-ones closed forms, an exact ``math.fsum`` sum and a
``fractions.Fraction`` brute force that must agree with the dgemm path within
the float64 bound, SwiGLU identities, and planted mistakes that must fail.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

GROUP = 64


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16): the bf16 value is the float32 whose
    top 16 bits are the pattern and whose low 16 bits are zero."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def activations_f64(x: np.ndarray) -> np.ndarray:
    """bf16 patterns (uint16), float32 or float64 activations -> float64 (exact)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError("activations are bf16 bit patterns (uint16), float32 or float64")


def unpack_codes(wq: np.ndarray, K: int) -> np.ndarray:
    """Codes q[n][k] in 0..15 from uint32 words, code k at bits 4*(k%8) of word k//8."""
    wq = np.asarray(wq, dtype=np.uint32)
    N = wq.shape[0]
    if wq.shape[1] * 8 != K:
        raise ValueError("wq must be [N][K/8]")
    k = np.arange(K)
    words = wq[:, k // 8]
    shifts = (4 * (k % 8)).astype(np.uint32)
    return ((words >> shifts[None, :]) & np.uint32(0xF)).astype(np.uint8).reshape(N, K)


def dequantize(wq, scales, biases, K: int) -> np.ndarray:
    """Float64 weights w[n][k] = S[n][k//64] * q[n][k] + B[n][k//64]."""
    q = unpack_codes(wq, K).astype(np.float64)
    s = bf16_to_f64(scales)
    b = bf16_to_f64(biases)
    g = np.arange(K) // GROUP
    return s[:, g] * q + b[:, g]


def matmul_rows(wq, scales, biases, x, cols=None) -> np.ndarray:
    """y[m][n] = sum_k w[n][k] x[m][k] in float64 (numpy dgemm on dequantized W).

    ``cols`` restricts the output to those columns n (for sampled checks of
    large matrices); the arithmetic per output is unchanged.
    """
    X = activations_f64(x)
    K = X.shape[1]
    if cols is not None:
        cols = np.asarray(cols)
        wq, scales, biases = wq[cols], scales[cols], biases[cols]
    W = dequantize(wq, scales, biases, K)
    return X @ W.T


def error_weight(wq, scales, biases, x, cols=None) -> np.ndarray:
    """A[m][n] = sum_k (|S| q + |B|)[n][k] * |x[m][k]|.

    The sum of absolute values of the 2K exact products that make up y; every
    rounding error bound of a summation order is a multiple of it.
    """
    X = np.abs(activations_f64(x))
    K = X.shape[1]
    if cols is not None:
        cols = np.asarray(cols)
        wq, scales, biases = wq[cols], scales[cols], biases[cols]
    q = unpack_codes(wq, K).astype(np.float64)
    g = np.arange(K) // GROUP
    Wabs = np.abs(bf16_to_f64(scales))[:, g] * q + np.abs(bf16_to_f64(biases))[:, g]
    return X @ Wabs.T


def _terms(wq, scales, biases, x_row_f64, n, K):
    """The 2K products s*q*x and b*x of output n. Each is exact in float64:
    s (8 significant bits) * q (4 bits) * x (8 bits for bf16, 24 for float32)
    and b (8 bits) * x fit in 53 bits."""
    q = unpack_codes(wq[n : n + 1], K)[0].astype(np.float64)
    s = bf16_to_f64(scales[n])
    b = bf16_to_f64(biases[n])
    g = np.arange(K) // GROUP
    return np.concatenate([s[g] * q * x_row_f64, b[g] * x_row_f64])


def matmul_rows_exact(wq, scales, biases, x, cols=None) -> np.ndarray:
    """Correctly rounded float64 y via ``math.fsum`` over the 2K exact products."""
    X = activations_f64(x)
    M, K = X.shape
    cols = np.arange(wq.shape[0]) if cols is None else np.asarray(cols)
    y = np.empty((M, len(cols)))
    for i in range(M):
        for j, n in enumerate(cols):
            y[i, j] = math.fsum(_terms(wq, scales, biases, X[i], int(n), K))
    return y


def matmul_rows_fraction(wq, scales, biases, x) -> list:
    """Exact rational y[m][n] by brute force: unpack, dequantize and sum with
    ``fractions.Fraction``, one code at a time (tiny shapes only)."""
    X = activations_f64(x)
    M, K = X.shape
    N = wq.shape[0]
    out = []
    for i in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                word = int(wq[n][k // 8])
                code = (word >> (4 * (k % 8))) & 0xF
                s = Fraction(float(bf16_to_f64(scales[n][k // GROUP])))
                b = Fraction(float(bf16_to_f64(biases[n][k // GROUP])))
                acc += (s * code + b) * Fraction(float(X[i][k]))
            row.append(acc)
        out.append(row)
    return out


def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a / (1 + exp(-a)) in float64 (overflow of exp gives -0/+0 correctly)."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu(a: np.ndarray, c: np.ndarray) -> np.ndarray:
    """SwiGLU of the paired projections: silu(w1 x) * (w3 x)."""
    return silu(a) * np.asarray(c, dtype=np.float64)
