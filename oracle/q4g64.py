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

Wider codes (PR #1514, "What changes": the MLX 4-, 6- and 8-bit checkpoints
are served as stored). The pages give no bit layout; the reading here is the
plain generalisation of the 4-bit one: the words of a row form one
little-endian bit stream (word j holds bits 32j .. 32j+31, bit 0 its least
significant) and code k of the row occupies bits ``bits*k .. bits*k+bits-1``
of it. 8-bit codes are then the bytes of each word in order; 6-bit codes
straddle word boundaries. Every function below takes ``bits`` (4, 6 or 8,
default 4); the dequantization and the sums do not change.

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


BITS = (4, 6, 8)


def words_per_row(K: int, bits: int = 4) -> int:
    if bits not in BITS:
        raise ValueError("bits must be 4, 6 or 8")
    if (K * bits) % 32:
        raise ValueError("K * bits must be a multiple of 32")
    return K * bits // 32


def unpack_codes(wq: np.ndarray, K: int, bits: int = 4) -> np.ndarray:
    """Codes q[n][k] in 0 .. 2^bits - 1 from uint32 words [N][K*bits/32]: code
    k occupies bits bits*k .. bits*k + bits - 1 of the row's bit stream (for 4
    bits: bits 4*(k%8) of word k//8, low nibble first)."""
    wq = np.asarray(wq, dtype=np.uint32)
    N = wq.shape[0]
    if wq.shape[1] != words_per_row(K, bits):
        raise ValueError("wq must be [N][K*bits/32]")
    pos = np.arange(K, dtype=np.int64) * bits  # first bit of each code
    w = pos // 32
    sh = (pos % 32).astype(np.uint64)
    # the two words a code can touch, joined as one 64-bit value (zero past the row)
    padded = np.concatenate([wq, np.zeros((N, 1), dtype=np.uint32)], axis=1).astype(np.uint64)
    pair = padded[:, w] | (padded[:, w + 1] << np.uint64(32))
    mask = np.uint64((1 << bits) - 1)
    return ((pair >> sh[None, :]) & mask).astype(np.uint8).reshape(N, K)


def dequantize(wq, scales, biases, K: int, bits: int = 4) -> np.ndarray:
    """Float64 weights w[n][k] = S[n][k//64] * q[n][k] + B[n][k//64]."""
    q = unpack_codes(wq, K, bits).astype(np.float64)
    s = bf16_to_f64(scales)
    b = bf16_to_f64(biases)
    g = np.arange(K) // GROUP
    return s[:, g] * q + b[:, g]


def matmul_rows(wq, scales, biases, x, cols=None, bits: int = 4) -> np.ndarray:
    """y[m][n] = sum_k w[n][k] x[m][k] in float64 (numpy dgemm on dequantized W).

    ``cols`` restricts the output to those columns n (for sampled checks of
    large matrices); the arithmetic per output is unchanged.
    """
    X = activations_f64(x)
    K = X.shape[1]
    if cols is not None:
        cols = np.asarray(cols)
        wq, scales, biases = wq[cols], scales[cols], biases[cols]
    W = dequantize(wq, scales, biases, K, bits)
    return X @ W.T


def error_weight(wq, scales, biases, x, cols=None, bits: int = 4) -> np.ndarray:
    """A[m][n] = sum_k (|S| q + |B|)[n][k] * |x[m][k]|.

    The sum of absolute values of the 2K exact products that make up y; every
    rounding error bound of a summation order is a multiple of it.
    """
    X = np.abs(activations_f64(x))
    K = X.shape[1]
    if cols is not None:
        cols = np.asarray(cols)
        wq, scales, biases = wq[cols], scales[cols], biases[cols]
    q = unpack_codes(wq, K, bits).astype(np.float64)
    g = np.arange(K) // GROUP
    Wabs = np.abs(bf16_to_f64(scales))[:, g] * q + np.abs(bf16_to_f64(biases))[:, g]
    return X @ Wabs.T


def _terms(wq, scales, biases, x_row_f64, n, K, bits=4):
    """The 2K products s*q*x and b*x of output n. Each is exact in float64:
    s (8 significant bits) * q (at most 8 bits) * x (8 bits for bf16, 24 for
    float32) and b (8 bits) * x fit in 53 bits."""
    q = unpack_codes(wq[n : n + 1], K, bits)[0].astype(np.float64)
    s = bf16_to_f64(scales[n])
    b = bf16_to_f64(biases[n])
    g = np.arange(K) // GROUP
    return np.concatenate([s[g] * q * x_row_f64, b[g] * x_row_f64])


def matmul_rows_exact(wq, scales, biases, x, cols=None, bits: int = 4) -> np.ndarray:
    """Correctly rounded float64 y via ``math.fsum`` over the 2K exact products."""
    X = activations_f64(x)
    M, K = X.shape
    cols = np.arange(wq.shape[0]) if cols is None else np.asarray(cols)
    y = np.empty((M, len(cols)))
    for i in range(M):
        for j, n in enumerate(cols):
            y[i, j] = math.fsum(_terms(wq, scales, biases, X[i], int(n), K, bits))
    return y


def matmul_rows_fraction(wq, scales, biases, x, bits: int = 4) -> list:
    """Exact rational y[m][n] by brute force: unpack, dequantize and sum with
    ``fractions.Fraction``, one code at a time (tiny shapes only). The code is
    read bit by bit from the row's words, independently of unpack_codes."""
    X = activations_f64(x)
    M, K = X.shape
    N = wq.shape[0]
    out = []
    for i in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                code = 0
                for t in range(bits):
                    pos = bits * k + t
                    code |= ((int(wq[n][pos // 32]) >> (pos % 32)) & 1) << t
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
