"""The accuracy figures the benchmark and the smoke check report (bf16-gap
ratio, bf16 flips, error over A), pinned on cases whose values are known."""

import numpy as np

from oracle.diagnostics import accuracy


def test_exact_result_has_no_error():
    y64 = np.array([1.0, -2.5, 3.0e-3, 7.0])
    a = accuracy(y64, y64, np.abs(y64) + 1.0)
    assert a["bf16_gap_ratio"] == 0.0 and a["bf16_flips"] == 0 and a["max_err_over_A"] == 0.0


def test_bf16_rounded_result_is_exactly_one_gap():
    rng = np.random.default_rng(0)
    y64 = rng.normal(0, 1, 1000)
    f = y64.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    yb = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    a = accuracy(yb, y64, np.ones_like(y64))
    assert abs(a["bf16_gap_ratio"] - 1.0) < 1e-6
    assert a["bf16_flips"] == 0


def test_flips_and_error_scale():
    y64 = np.array([1.0, 1.0, 1.0, 1.0])
    y = y64 + np.array([0.0, 2.0 ** -7, 0.0, -(2.0 ** -6)])  # two outputs a bf16 ulp or more away
    A = np.array([1.0, 2.0, 4.0, 8.0])
    a = accuracy(y, y64, A)
    assert a["bf16_flips"] == 2
    assert a["max_err_over_A"] == 2.0 ** -7 / 2.0
    assert np.isclose(a["rms_err_over_A"], np.sqrt(((2.0 ** -8) ** 2 + (2.0 ** -9) ** 2) / 4))
