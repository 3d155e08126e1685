"""The bound of the device SwiGLU gate and its planted control, on the CPU.

The device silu (float32) forms exp(-a) as 2^(t + t_lo), with t + t_lo =
-a * log2(e) carried in two floats, then 1 + e, a reciprocal and a product;
its stated error is 7 * 2^-24 relative wherever |silu(a)| > 2^-100
(TensorFold PR #1696, "What it adds" > Kernels without DPAS: an FP64 op test
and a planted control per kernel). A float32 model of that evaluation, with
correctly rounded exp2 and reciprocal, stays inside the bound on the op
test's arguments; the same model without the two-float argument (the
rounding error of -a * log2(e) left in the exponent) must leave it. The GPU
op test (test_gpu_silu.py) checks the device outputs against the same bound.
"""

import numpy as np

import oracle
from tests import silu_cases
from tests.tolerance import SILU_REL, silu_bound

F32, F64 = np.float32, np.float64
LOG2E = F32(float.fromhex("0x1.715476p+0"))
LOG2E_TAIL = F32(float.fromhex("0x1.4ae0c0p-26"))
LN2 = F32(float.fromhex("0x1.62e430p-1"))


def case_arguments():
    """Gate arguments a = fl32(s * q + b) of the op test's columns."""
    s_bits, q, b_bits = silu_cases.cases()
    s = oracle.bf16_to_f64(s_bits)
    b = oracle.bf16_to_f64(b_bits)
    return (s * q.astype(F64) + b).astype(F32)  # exact in float64, one rounding


def silu_f32_model(a, two_float=True):
    a = np.asarray(a, dtype=F32)
    ac = np.clip(a, F32(-80.0), F32(88.0)).astype(F32)
    t = (-ac * LOG2E).astype(F32)
    e = np.exp2(t.astype(F64)).astype(F32)
    if two_float:
        lo = ((-ac).astype(F64) * F64(LOG2E) - t.astype(F64)).astype(F32)  # fma: exact, one rounding
        t_lo = (lo + (-ac * LOG2E_TAIL).astype(F32)).astype(F32)
        corr = (t_lo * LN2).astype(F32)
        e = (e.astype(F64) * corr.astype(F64) + e.astype(F64)).astype(F32)  # fma
    d = (F32(1.0) + e).astype(F32)
    r = (1.0 / d.astype(F64)).astype(F32)
    z = (a.astype(F64) * r.astype(F64)).astype(F32)
    return np.where(a < F32(-80.0), F32(-0.0), z)


def excess(z, a):
    """Largest |z - silu64(a)| / bound; at most 1 inside the stated bound."""
    err = np.abs(z.astype(F64) - oracle.silu(a.astype(F64)))
    return float(np.max(err / silu_bound(a)))


def test_cases_span_the_argument_range():
    a = case_arguments().astype(F64)
    assert np.all(np.isfinite(a))
    assert a.min() < -1e30 and a.max() > 1e30
    assert np.any(np.abs(a) < 2.0 ** -120) and np.any((a > 0) & (a < 1e-30)) and np.any((a < 0) & (a > -1e-30))
    for p in (-80.0, 88.0):
        near = np.abs(a - p) <= 2.0 ** -10
        assert np.sum(near & (a < p)) > 10 and np.sum(near & (a > p)) > 10 and np.any(a == p)
    assert len(np.unique(a)) > 15000


def test_model_of_the_device_silu_is_inside_its_bound():
    a = case_arguments()
    r = excess(silu_f32_model(a), a)
    assert r <= 1.0, r
    # and it uses a good part of it, so the bound is not vacuous here
    assert r > 0.2, r


def test_planted_single_float_argument_fails_the_bound():
    a = case_arguments()
    r = excess(silu_f32_model(a, two_float=False), a)
    assert r > 1.0, r


def test_bound_is_the_stated_relative_one():
    a = np.array([1.0, -1.0, 10.0, -10.0], dtype=F32)
    assert np.allclose(silu_bound(a), SILU_REL * np.abs(oracle.silu(a.astype(F64))), rtol=0, atol=0)
    assert silu_bound(np.array([-200.0], dtype=F32))[0] == 2.0 ** -100


def test_case_arguments_are_exact_in_float32():
    """s * q + b needs no rounding in float32 for any case, so the decode
    fold (one fused multiply-add) and the window's matrix-core bias step
    (whatever its rounding mode) both produce exactly this a."""
    s_bits, q, b_bits = silu_cases.cases()
    exact = oracle.bf16_to_f64(s_bits) * q.astype(F64) + oracle.bf16_to_f64(b_bits)
    assert np.array_equal(exact.astype(F32).astype(F64), exact)
