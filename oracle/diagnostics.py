"""Op-level accuracy figures of a result against the float64 oracle.

TEST INFRASTRUCTURE, like the rest of ``oracle/``: the tests, the smoke check
and the benchmark's CPU-baseline leg report these numbers; nothing gates on
them (the parity gate is the stated bound in tests/tolerance.py).

The figures are the ones the pages report for their kernels (TensorFold PR
#1696, "Checks" > Forward against float64: a layer's error as a multiple of
the bf16 gap; later revision, "Checks" > pgemm against float64: the float32
error and the count of bf16 flips):

* bf16-gap ratio  ||y - y64||_2 / ||bf16(y64) - y64||_2: the error against
  the error of rounding the exact result to bf16 (well below 1 for a float32
  computation);
* bf16 flips: outputs whose round-to-nearest-even bf16 differs from that of
  the exact result (near-ties may legitimately flip);
* max and RMS of |y - y64| / A, with A = sum |w| |x| the scale of every
  rounding bound.
"""

from __future__ import annotations

import numpy as np


def _bf16_rne(v: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bf16 (RNE), returned as float64 values."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def accuracy(y, y64, A) -> dict:
    """The figures above for a result y (any float dtype) against the exact
    y64 with error weight A (same shape)."""
    y = np.asarray(y, dtype=np.float64)
    y64 = np.asarray(y64, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    err = y - y64
    gap = _bf16_rne(y64) - y64
    gap_norm = float(np.linalg.norm(gap))
    rel = np.abs(err) / np.where(A > 0, A, np.inf)
    return {
        "bf16_gap_ratio": float(np.linalg.norm(err)) / gap_norm if gap_norm > 0 else 0.0,
        "bf16_flips": int(np.count_nonzero(_bf16_rne(y) != _bf16_rne(y64))),
        "outputs": int(y.size),
        "max_err_over_A": float(np.max(rel)) if rel.size else 0.0,
        "rms_err_over_A": float(np.sqrt(np.mean(rel * rel))) if rel.size else 0.0,
    }
