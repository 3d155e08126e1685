"""Stated error bounds between the GPU kernels and the float64 oracle.

Every product the kernels form is exact in float32 (a bf16 activation times
a code of at most 8 significant bits, bf16 times 1, a bf16 bias times a bf16
piece); the scale enters through a fused multiply-add. Rounding happens only
in additions, so the error of a fixed summation order is at most n * u * A,
where A = sum of |products| (the oracle's ``error_weight``), u = 2^-23 (twice
the float32 unit roundoff, which also covers truncating rather than nearest
rounding inside a matrix core) and n bounds the roundings on any path from a
term to the result. Each rounding is at most u times the magnitude of the
partial sum it rounds, which is at most the running part of A.

The count n depends on the kernel family's order (TensorFold PR #1696, later
revision, "What it adds": decode keeps its own kernels and the prompt GEMM
uses a different summation order):

In-group (both orders): a group's code sum P_g = sum q*x and activation sum
S_g = sum x are each one chain of 64 terms, at most 64 roundings. The errors
of P_g reach the result multiplied by s and those of S_g multiplied by b, so
they fall on the disjoint parts sum |s| q |x| and sum |b| |x| of A: 64 in
all, not 64 for each. Float32 activations are split by truncation into three
bf16 pieces h + m + l = x that all share the sign of x, so |h| + |m| + |l| =
|x|: the three piece chains together still count 64, plus the two additions
that join the pieces.

Decode (qmv_rows, qmv_w13_swiglu, the one-launch FFN step, the fused q/k/v
epilogue): per group the fold acc <- fma(s, P, fma(b, S, acc)) rounds twice
(block FP8: acc <- fma(s, P, acc), once); the parts of the 256-wide segments
are joined in ascending order, one addition per segment.

Window (qmm_window): per group the fold acc <- fma(s, P, acc) rounds once;
the bias terms b_g * piece of each chunk of 8 groups enter through two
matrix-core steps with the running total as their accumulator input. Only
non-zero terms can make an addition inexact, and each group contributes at
most 3 pieces, so at most 3 roundings per group there (block FP8 has no bias
step). 6 per group are allowed.

Eight of slack cover second-order terms. Denormal flushing is covered by an
absolute floor.
"""

import numpy as np

U = 2.0 ** -23
FLOOR = 2.0 ** -100
ORDERS = ("decode", "window")
FORMATS = ("affine", "fp8")


def units(K: int, x_dtype: str = "bf16", *, order: str, fmt: str = "affine") -> int:
    """Rounding count n of the bound n * u * A for one kernel family."""
    if order not in ORDERS:
        raise ValueError(f"order must be one of {ORDERS}")
    if fmt not in FORMATS:
        raise ValueError(f"fmt must be one of {FORMATS}")
    if x_dtype not in ("bf16", "f32"):
        raise ValueError("x_dtype must be bf16 or f32")
    G = K // 64
    in_group = 64 + (2 if x_dtype == "f32" else 0)
    if order == "decode":
        per_group = 2 if fmt == "affine" else 1
        return in_group + per_group * G + -(-G // 4) + 8
    if x_dtype != "bf16":
        raise ValueError("the prompt GEMM takes bf16 activations only")
    per_group = 6 if fmt == "affine" else 1
    return in_group + per_group * G + 8


def tol(A: np.ndarray, K: int, x_dtype: str = "bf16", *, order: str, fmt: str = "affine") -> np.ndarray:
    return units(K, x_dtype, order=order, fmt=fmt) * U * np.asarray(A) + FLOOR


def tol_loosest(A: np.ndarray, K: int, fmt: str = "affine") -> np.ndarray:
    """The larger of the two orders' bounds for bf16 activations: a planted
    mistake must exceed every gate that could be applied to the data."""
    n = max(units(K, order=o, fmt=fmt) for o in ORDERS)
    return n * U * np.asarray(A) + FLOOR


# The device silu's stated relative error (exp on a two-float argument, the
# hardware exp2 and reciprocal): 3 + 1 + 2 + 1 units of 2^-24.
SILU_REL = 7.0 * 2.0 ** -24
# Below this magnitude of the exact value the bound is absolute.
SILU_FLOOR = 2.0 ** -100


def silu_bound(a64) -> np.ndarray:
    """Bound on |silu_dev(a) - silu(a)| for a float32 argument a (exact in
    float64): SILU_REL relative, or SILU_FLOOR absolute where |silu(a)| is
    below it."""
    from oracle import silu  # oracle: float64 silu

    return np.maximum(SILU_REL * np.abs(silu(np.asarray(a64, dtype=np.float64))), SILU_FLOOR)


def tol_swiglu(a64, c64, Ta, Tc) -> np.ndarray:
    """Bound on |fl(silu(a_hat) * c_hat) - silu(a64) * c64|.

    |silu'| <= 1.0999 everywhere; the kernels' float32 silu is within
    7 * 2^-24 < 2^-21 relative wherever |silu| > 2^-100 (below that the error
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
