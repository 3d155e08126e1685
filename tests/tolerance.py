"""Stated error bounds between the GPU kernels and the float64 oracle.

Every product the kernels form is exact in float32 (bf16 x times a 4-bit
integer code, bf16 x times 1, bf16 scale/bias times an fp32 sum is fused).
Rounding happens only in additions, so the error of a fixed summation order
with n roundings is at most gamma_n * A, where A = sum of |products| (the
oracle's ``error_weight``) and gamma_n <= n * u, with u = 2^-23 (twice the
float32 unit roundoff, which also covers truncating rather than nearest
rounding inside a matrix core). The count n covers both kernel orders:

* up to 64 (bf16 x) or 192 (float32 x split into three exact bf16 pieces)
  roundings inside one 64-wide group's matrix-core dot product, and as many
  for that group's activation sum;
* per group: up to 2 roundings in the decode fold
  acc <- fma(s, P, fma(b, S, acc)), or 1 in the prompt GEMM's fold
  acc <- fma(s, P, acc) plus up to 4 inside the matrix-core bias product
  sum_g b_g * S_g (4 slots per group) and its chaining: 6 * K/64 allowed;
* one addition per 256-wide k segment when segments are combined;
* 16 of slack.

Denormal flushing adds at most a tiny absolute floor.
"""

import numpy as np

U = 2.0 ** -23
FLOOR = 2.0 ** -100


def units(K: int, x_dtype: str = "bf16") -> int:
    G = K // 64
    piece = 1 if x_dtype == "bf16" else 3
    segments = -(-G // 4)
    return 128 * piece + 6 * G + segments + 16


def tol(A: np.ndarray, K: int, x_dtype: str = "bf16") -> np.ndarray:
    return units(K, x_dtype) * U * np.asarray(A) + FLOOR


def tol_swiglu(a64, c64, Ta, Tc) -> np.ndarray:
    """Bound on |fl(silu(a_hat) * c_hat) - silu(a64) * c64|.

    |silu'| <= 1.0999 everywhere; the kernels' float32 silu is within
    7 * 2^-24 < 2^-21 relative wherever |silu| > 2^-100 (exp via the hardware
    exp2 on a two-float argument, hardware reciprocal; below that the error
    is under the absolute floor); the final product adds one rounding.
    """
    from oracle import silu  # oracle: float64 silu

    s64 = np.abs(silu(a64))
    c = np.abs(c64)
    Es = 1.1 * Ta + 2.0 ** -21 * (s64 + 1.1 * Ta)
    return Es * (c + Tc) + s64 * Tc + 2.0 ** -23 * (s64 + Es) * (c + Tc) + FLOOR


def tol_bf16_out(y64, T) -> np.ndarray:
    """Extra half-ulp (relative 2^-9, taken as 2^-8) for a bf16 output."""
    return T + 2.0 ** -8 * (np.abs(y64) + T) + 2.0 ** -126
