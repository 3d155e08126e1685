"""The C-ABI library: it loads, exports every function include/q4g64.h
declares, and rejects bad arguments on the host with the documented status
codes before anything reaches a device (no GPU needed: these calls fail
validation and never enqueue)."""

import ctypes
import math
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import bit_weight_only_q4g64_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4g64.h")

FAKE = 0x10000  # aligned non-null address; only passed where validation fails first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return [n for n in names if n not in ("if", "defined")]


def test_header_declares_the_boundary():
    names = set(_declared())
    for must in ("pack_q4g64", "qmv_rows", "qmv_w13_swiglu", "qmm_window", "qmm_cut", "q4g64_packed_bytes", "q4_last_error"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = q4.lib()
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(q4._SIGNATURES)
    assert lib.q4g64_abi_version() == 4


def test_packed_bytes():
    assert q4.packed_bytes(512, 256) == 512 * 256 * 9 // 16
    assert q4.packed_bytes(8192, 2048) == 9437184
    assert q4.packed_bytes(64, 192) == 4 * 2 * 1152  # odd group count pads the last pair
    for bad in ((0, 64), (64, 0), (100, 64), (64, 100), (-64, 64), (1 << 31, 64)):
        assert q4.packed_bytes(*bad) == 0


def _rc(name, *args):
    lib = q4.lib()
    rc = getattr(lib, name)(*args)
    return rc, lib.q4_last_error().decode()


@pytest.mark.parametrize("N,K", [(100, 256), (512, 100), (0, 256), (512, -64), (48, 256)])
def test_bad_shapes_rejected(N, K):
    rc, msg = _rc("qmv_rows", FAKE, N, K, FAKE, q4.Q4_BF16, 256, 1, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL and "multiples of 64" in msg
    rc, _ = _rc("pack_q4g64", FAKE, FAKE, FAKE, N, K, FAKE, None)
    assert rc == q4.Q4_EINVAL
    rc, _ = _rc("qmm_window", FAKE, None, N, K, FAKE, 256, 4, FAKE, q4.Q4_F32, 512, None)
    assert rc == q4.Q4_EINVAL


@pytest.mark.parametrize("R", [0, 17, -1])
def test_row_count_rejected(R):
    rc, msg = _rc("qmv_rows", FAKE, 512, 256, FAKE, q4.Q4_BF16, 256, R, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL and "R=" in msg
    rc, _ = _rc("qmv_w13_swiglu", FAKE, FAKE, 512, 256, FAKE, 256, R, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL


def test_null_and_misaligned_pointers_rejected():
    rc, msg = _rc("qmv_rows", None, 512, 256, FAKE, q4.Q4_BF16, 256, 1, FAKE, 512, None)
    assert rc == q4.Q4_EALIGN and "NULL" in msg
    rc, msg = _rc("qmv_rows", FAKE + 8, 512, 256, FAKE, q4.Q4_BF16, 256, 1, FAKE, 512, None)
    assert rc == q4.Q4_EALIGN and "aligned" in msg
    rc, _ = _rc("qmv_rows", FAKE, 512, 256, FAKE + 2, q4.Q4_BF16, 256, 1, FAKE, 512, None)
    assert rc == q4.Q4_EALIGN
    rc, _ = _rc("qmm_window", FAKE, FAKE + 4, 512, 256, FAKE, 256, 4, FAKE, q4.Q4_F32, 512, None)
    assert rc == q4.Q4_EALIGN


def test_strides_and_dtypes_rejected():
    # ldx < K
    rc, _ = _rc("qmv_rows", FAKE, 512, 256, FAKE, q4.Q4_BF16, 128, 1, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL
    # ldx keeps rows 16-byte aligned only in multiples of 8 bf16 / 4 float32
    rc, _ = _rc("qmv_rows", FAKE, 512, 256, FAKE, q4.Q4_BF16, 260, 1, FAKE, 512, None)
    assert rc == q4.Q4_EALIGN
    rc, _ = _rc("qmv_rows", FAKE, 512, 256, FAKE, q4.Q4_F32, 258, 1, FAKE, 512, None)
    assert rc == q4.Q4_EALIGN
    # ldy < N
    rc, _ = _rc("qmv_rows", FAKE, 512, 256, FAKE, q4.Q4_BF16, 256, 1, FAKE, 500, None)
    assert rc == q4.Q4_EINVAL
    # unknown dtypes
    rc, _ = _rc("qmv_rows", FAKE, 512, 256, FAKE, 7, 256, 1, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL
    rc, _ = _rc("qmm_window", FAKE, None, 512, 256, FAKE, 256, 4, FAKE, 9, 512, None)
    assert rc == q4.Q4_EINVAL


def test_planes_arguments_rejected():
    """Q4_BF16X3 planes: the planes dtype is accepted only as a decode input, with bf16 stride rules; the planes
    output of the fused SwiGLU checks its width, pointer and 16-byte row alignment."""
    rc, _ = _rc("qmv_rows", FAKE, 512, 256, FAKE, 4, 256, 1, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL
    rc, _ = _rc("qmv_rows", FAKE, 512, 256, FAKE, q4.Q4_BF16X3, 260, 1, FAKE, 512, None)
    assert rc == q4.Q4_EALIGN  # 520-byte rows
    rc, _ = _rc("qmv_rows_qg64", 8, FAKE, 512, 256, FAKE, q4.Q4_BF16X3, 128, 1, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL  # ldx < K
    rc, _ = _rc("qmm_window", FAKE, None, 512, 256, FAKE, 256, 4, FAKE, q4.Q4_BF16X3, 512, None)
    assert rc == q4.Q4_EINVAL  # not a window output type
    rc, _ = _rc("qmv_w13_swiglu_x3", 5, FAKE, FAKE, 1024, 256, FAKE, 256, 1, FAKE, 1024, None)
    assert rc == q4.Q4_EINVAL
    rc, msg = _rc("qmv_w13_swiglu_x3", 4, FAKE, FAKE, 1024, 256, FAKE, 256, 1, FAKE, 1000, None)
    assert rc == q4.Q4_EINVAL and "ldz" in msg
    rc, msg = _rc("qmv_w13_swiglu_x3", 4, FAKE, FAKE, 1024, 256, FAKE, 256, 1, FAKE, 1028, None)
    assert rc == q4.Q4_EALIGN and "ldz" in msg
    rc, _ = _rc("qmv_w13_swiglu_x3", 6, FAKE, FAKE, 1024, 256, FAKE, 256, 1, None, 1024, None)
    assert rc == q4.Q4_EALIGN
    rc, _ = _rc("qmv_w13_swiglu_x3_fp8b", FAKE, FAKE, 1024, 256, FAKE, 256, 1, FAKE + 2, 1024, None)
    assert rc == q4.Q4_EALIGN
    rc, _ = _rc("qmv_w13_swiglu_x3_fp8b", FAKE, FAKE, 1024, 256, FAKE, 256, 17, FAKE, 1024, None)
    assert rc == q4.Q4_EINVAL


def test_tiled_planes_bytes():
    """Q4_BF16X3T: K/64 groups x (1, 2 or 4 row tiles) x 2 KiB; 0 for invalid K or R."""
    f = q4.lib().q4g64_x3t_bytes
    assert f(2048, 1) == 32 * 1 * 2048
    assert f(2048, 4) == 32 * 1 * 2048
    assert f(2048, 5) == 32 * 2 * 2048
    assert f(8192, 9) == 128 * 4 * 2048
    assert f(16384, 16) == 256 * 4 * 2048
    for K, R in ((100, 1), (2048, 0), (2048, 17), (16448, 1), (0, 1), (-64, 1)):
        assert f(K, R) == 0, (K, R)


def test_tiled_planes_arguments_rejected():
    """Q4_BF16X3T is a decode input without a row stride (ldx must equal K) and never a window output type; the
    tiled output of the fused SwiGLU checks its bits, pointer, row count and the width the next matvec can take."""
    rc, msg = _rc("qmv_rows", FAKE, 512, 256, FAKE, q4.Q4_BF16X3T, 264, 1, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL and "ldx" in msg
    rc, _ = _rc("qmv_rows_fp8b", FAKE, 512, 256, FAKE, q4.Q4_BF16X3T, 128, 4, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL
    rc, _ = _rc("qmv_rows", FAKE, 512, 256, FAKE + 8, q4.Q4_BF16X3T, 256, 4, FAKE, 512, None)
    assert rc == q4.Q4_EALIGN
    rc, _ = _rc("qmm_window", FAKE, None, 512, 256, FAKE, 256, 4, FAKE, q4.Q4_BF16X3T, 512, None)
    assert rc == q4.Q4_EINVAL
    rc, _ = _rc("qmv_w13_swiglu_x3t", 5, FAKE, FAKE, 1024, 256, FAKE, 256, 1, FAKE, None)
    assert rc == q4.Q4_EINVAL
    rc, _ = _rc("qmv_w13_swiglu_x3t", 4, FAKE, FAKE, 1024, 256, FAKE, 256, 1, None, None)
    assert rc == q4.Q4_EALIGN
    rc, _ = _rc("qmv_w13_swiglu_x3t", 8, FAKE, FAKE, 1024, 256, FAKE, 256, 1, FAKE + 2, None)
    assert rc == q4.Q4_EALIGN
    rc, _ = _rc("qmv_w13_swiglu_x3t", 4, FAKE, FAKE, 1024, 256, FAKE, 256, 17, FAKE, None)
    assert rc == q4.Q4_EINVAL
    rc, _ = _rc("qmv_w13_swiglu_x3t", 4, FAKE, FAKE, 16448, 256, FAKE, 256, 1, FAKE, None)
    assert rc == q4.Q4_EUNSUPPORTED
    rc, _ = _rc("qmv_w13_swiglu_x3t_fp8b", FAKE, FAKE, 1024, 256, FAKE, 256, 0, FAKE, None)
    assert rc == q4.Q4_EINVAL


def test_window_counts_rejected():
    rc, _ = _rc("qmm_window", FAKE, None, 512, 256, FAKE, 256, 0, FAKE, q4.Q4_F32, 512, None)
    assert rc == q4.Q4_EINVAL
    arr = (ctypes.c_int64 * 3)(17, 0, 5)
    rc, msg = _rc("qmm_cut", FAKE, None, 512, 256, FAKE, 256, arr, 3, FAKE, q4.Q4_F32, 512, None)
    assert rc == q4.Q4_EINVAL and "window 1" in msg
    rc, _ = _rc("qmm_cut", FAKE, None, 512, 256, FAKE, 256, None, 0, FAKE, q4.Q4_F32, 512, None)
    assert rc == q4.Q4_EINVAL


def test_decode_k_limits():
    rc, msg = _rc("qmv_rows", FAKE, 512, 32768, FAKE, q4.Q4_BF16, 32768, 1, FAKE, 512, None)
    assert rc == q4.Q4_EUNSUPPORTED and "16384" in msg
    rc, msg = _rc("qmv_w13_swiglu", FAKE, FAKE, 512, 16384, FAKE, 16384, 1, FAKE, 512, None)
    assert rc == q4.Q4_EUNSUPPORTED and "8192" in msg


def test_binding_refuses_host_tensors():
    import torch

    x = torch.zeros((1, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        q4.qmv_rows(torch.zeros(10, dtype=torch.uint8), 512, 256, x)


def test_ffn_work_bytes():
    # the error word and the call counter block (4352 B), the one-launch step's
    # tagged z copy for up to 2 rows (8 B per value) and lower-half sums (64
    # lanes x 8 B per 16-column tile of w2); then the fragment-ordered planes
    # the two-call step hands over, for up to 16 rows (4 piece slots of 2 B
    # per row and k). No dependence on R.
    def size(N1, N2):
        head = 4352 + 2 * N1 * 8 + (N2 // 16) * 512
        return (head + 255) // 256 * 256 + N1 * 4 * 2 * 16
    for R in (1, 2, 3, 4, 5, 16):
        assert q4.ffn_work_bytes(8192, 2048, R) == size(8192, 2048) == 1249536
    assert q4.ffn_work_bytes(64, 64, 1) == size(64, 64)
    assert q4.ffn_work_bytes(192, 128, 3) == size(192, 128)
    for bad in ((0, 64, 1), (100, 64, 1), (8192, 64, 0), (8192, 64, 17), (32768, 64, 1), (8192, 100, 1), (8192, 0, 1)):
        assert q4.ffn_work_bytes(*bad) == 0


def _ffn(N1=8192, K1=2048, N2=2048, ldx=2048, R=1, ldz=8192, ldy=2048, work=FAKE, p=FAKE):
    return _rc("qmv_ffn", p, FAKE, FAKE, N1, K1, N2, FAKE, ldx, R, FAKE, ldz, FAKE, ldy, work, None)


def test_ffn_rejects_bad_arguments():
    assert _ffn(N1=8100)[0] == q4.Q4_EINVAL
    assert _ffn(N2=100)[0] == q4.Q4_EINVAL
    assert _ffn(K1=0)[0] == q4.Q4_EINVAL
    for R in (0, 17):
        rc, msg = _ffn(R=R)
        assert rc == q4.Q4_EINVAL and "R=" in msg
    assert _ffn(p=None)[0] == q4.Q4_EALIGN
    rc, msg = _ffn(work=None)
    assert rc == q4.Q4_EALIGN and "work" in msg
    rc, msg = _ffn(work=FAKE + 16)
    assert rc == q4.Q4_EALIGN and "work" in msg
    assert _ffn(ldx=1024)[0] == q4.Q4_EINVAL
    assert _ffn(ldz=4096)[0] == q4.Q4_EINVAL
    assert _ffn(ldy=1024)[0] == q4.Q4_EINVAL
    rc, msg = _ffn(K1=8192, ldx=8192)
    assert rc == q4.Q4_EUNSUPPORTED and "4096" in msg
    rc, msg = _ffn(N1=16384, ldz=16384)
    assert rc == q4.Q4_EUNSUPPORTED and "8192" in msg


def test_wide_packed_bytes():
    # 256 * bits bytes of codes plus 128 of scale/bias per column tile and group pair
    assert q4.packed_bytes(512, 256, bits=4) == q4.packed_bytes(512, 256)
    assert q4.packed_bytes(512, 256, bits=8) == 32 * 2 * (2048 + 128)
    assert q4.packed_bytes(512, 256, bits=6) == 32 * 2 * (1536 + 128)
    assert q4.packed_bytes(8192, 2048, bits=8) == 8192 * 2048 + 8192 * 32 * 4
    assert q4.packed_bytes(64, 192, bits=6) == 4 * 2 * (1536 + 128)
    for bits in (0, 3, 5, 7, 16):
        assert q4.packed_bytes(512, 256, bits=bits) == 0


@pytest.mark.parametrize("bits", [0, 5, 7, 16])
def test_wide_calls_reject_bad_bits(bits):
    rc, msg = _rc("pack_qg64", bits, FAKE, FAKE, FAKE, 512, 256, FAKE, None)
    assert rc == q4.Q4_EINVAL and "bits" in msg
    rc, msg = _rc("unpack_qg64", bits, FAKE, 512, 256, FAKE, FAKE, FAKE, None)
    assert rc == q4.Q4_EINVAL and "bits" in msg
    rc, msg = _rc("qmv_rows_qg64", bits, FAKE, 512, 256, FAKE, q4.Q4_BF16, 256, 1, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL and "bits" in msg
    rc, msg = _rc("qmv_w13_swiglu_qg64", bits, FAKE, FAKE, 512, 256, FAKE, 256, 1, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL and "bits" in msg


@pytest.mark.parametrize("bits", [6, 8])
def test_wide_calls_validate_like_q4(bits):
    rc, msg = _rc("qmv_rows_qg64", bits, FAKE, 100, 256, FAKE, q4.Q4_BF16, 256, 1, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL and "multiples of 64" in msg
    rc, _ = _rc("qmv_rows_qg64", bits, FAKE, 512, 256, FAKE, q4.Q4_BF16, 256, 17, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL
    rc, _ = _rc("qmv_rows_qg64", bits, None, 512, 256, FAKE, q4.Q4_BF16, 256, 1, FAKE, 512, None)
    assert rc == q4.Q4_EALIGN
    rc, _ = _rc("qmv_w13_swiglu_qg64", bits, FAKE, FAKE, 512, 16384, FAKE, 16384, 1, FAKE, 512, None)
    assert rc == q4.Q4_EUNSUPPORTED
    rc, _ = _rc("pack_qg64", bits, FAKE + 8, FAKE, FAKE, 512, 256, FAKE, None)
    assert rc == q4.Q4_EALIGN


def test_window_cost_interpolation():
    us = [5.0, 6.0, 8.0, 9.0, 13.0]
    for R, c in zip((1, 2, 4, 8, 16), us):
        assert q4.window_cost(us, R) == c
    assert q4.window_cost(us, 3) == 7.0
    # the timed row counts read back exactly even next to a much larger entry
    far = [203.853515625, 3.8175501823425293, 4.233449935913086, 5.397349834442139, 9.718850135803223]
    for R, c in zip(q4.WINDOW_COST_ROWS, far):
        assert q4.window_cost(far, R) == np.float32(c)
    assert q4.window_cost(us, 6) == 8.5
    assert q4.window_cost(us, 12) == 11.0
    assert abs(q4.window_cost(us, 5) - 8.25) < 1e-6
    for R in (0, -1, 17, 100):
        assert math.isnan(q4.window_cost(us, R))
    assert math.isnan(q4.lib().qmv_window_cost(None, 4))


def test_window_costs_rejects_bad_arguments():
    out = (ctypes.c_float * 5)()
    args = (4, FAKE, 512, 256, FAKE, q4.Q4_BF16, 256, FAKE, 512)
    rc, msg = _rc("qmv_window_costs", *args, 10, None, None)
    assert rc == q4.Q4_EINVAL and "us_out" in msg
    for reps in (0, 10001):
        rc, msg = _rc("qmv_window_costs", *args, reps, ctypes.addressof(out), None)
        assert rc == q4.Q4_EINVAL and "reps" in msg
    rc, msg = _rc("qmv_window_costs", 5, *args[1:], 10, ctypes.addressof(out), None)
    assert rc == q4.Q4_EINVAL and "bits" in msg
    rc, _ = _rc("qmv_window_costs", 4, FAKE, 100, 256, FAKE, q4.Q4_BF16, 256, FAKE, 512, 10, ctypes.addressof(out), None)
    assert rc == q4.Q4_EINVAL
    rc, _ = _rc("qmv_window_costs", 4, FAKE, 512, 256, FAKE, q4.Q4_BF16, 256, FAKE, 100, 10, ctypes.addressof(out), None)
    assert rc == q4.Q4_EINVAL  # ldy < N


def test_fp8_packed_bytes_and_rejections():
    assert q4.fp8b_packed_bytes(512, 256) == q4.packed_bytes(512, 256, bits=8)
    assert q4.fp8b_packed_bytes(100, 256) == 0
    rc, _ = _rc("pack_fp8b", FAKE, FAKE, 100, 256, FAKE, None)
    assert rc == q4.Q4_EINVAL
    rc, _ = _rc("pack_fp8b", FAKE + 8, FAKE, 512, 256, FAKE, None)
    assert rc == q4.Q4_EALIGN
    rc, _ = _rc("pack_fp8b", FAKE, FAKE + 2, 512, 256, FAKE, None)
    assert rc == q4.Q4_EALIGN
    rc, _ = _rc("qmv_rows_fp8b", FAKE, 512, 256, FAKE, q4.Q4_BF16, 256, 17, FAKE, 512, None)
    assert rc == q4.Q4_EINVAL
    rc, _ = _rc("qmm_window_fp8b", FAKE, None, 512, 256, FAKE, 256, 0, FAKE, q4.Q4_F32, 512, None)
    assert rc == q4.Q4_EINVAL
    rc, _ = _rc("qmv_window_costs", 9, FAKE, 512, 256, FAKE, q4.Q4_BF16, 256, FAKE, 512, 10, FAKE, None)
    assert rc == q4.Q4_EINVAL  # the public width argument takes 4, 6 or 8 only


def _rope(**kw):
    base = dict(pos=FAKE, n_q_heads=32, n_kv_heads=8, rot_dims=64, theta=10000.0, gamma_q=None, gamma_k=None, eps=1e-6,
                q_out=FAKE, ldq=2048, k_cache=FAKE, v_cache=FAKE, cache_dtype=q4.Q4_F32, ring_len=64)
    base.update(kw)
    return q4.RopeKv(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=0), q4.Q4_EINVAL), (dict(n_kv_heads=0), q4.Q4_EINVAL), (dict(rot_dims=3), q4.Q4_EINVAL),
    (dict(rot_dims=66), q4.Q4_EINVAL), (dict(theta=0.0), q4.Q4_EINVAL), (dict(theta=float("inf")), q4.Q4_EINVAL),
    (dict(eps=-1.0), q4.Q4_EINVAL), (dict(cache_dtype=7), q4.Q4_EINVAL), (dict(ring_len=0), q4.Q4_EINVAL),
    (dict(ldq=100), q4.Q4_EINVAL), (dict(pos=None), q4.Q4_EALIGN), (dict(q_out=FAKE + 2), q4.Q4_EALIGN),
    (dict(k_cache=None), q4.Q4_EALIGN), (dict(gamma_q=FAKE + 1), q4.Q4_EALIGN),
    (dict(cache_row_stride=-1), q4.Q4_EINVAL), (dict(cache_row_stride=64 * 8 * 64 - 1), q4.Q4_EINVAL)])
def test_rope_args_rejected(kw, code):
    a = _rope(**kw)
    rc, _ = _rc("rope_kv_store", FAKE, 3072, 1, ctypes.addressof(a), None)
    assert rc == code
    rc, _ = _rc("qmv_qkv_rope", 4, FAKE, 2048, FAKE, 2048, 1, ctypes.addressof(a), None)
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(n_gate_heads=-1), q4.Q4_EINVAL), (dict(n_gate_heads=4097, gate_out=FAKE, ldg=4097 * 64), q4.Q4_EINVAL),
    (dict(n_gate_heads=32, gate_out=FAKE, ldg=100), q4.Q4_EINVAL), (dict(n_gate_heads=32, gate_out=None, ldg=2048), q4.Q4_EALIGN),
    (dict(n_gate_heads=32, gate_out=FAKE + 2, ldg=2048), q4.Q4_EALIGN)])
def test_rope_gate_args_rejected(kw, code):
    a = _rope(**kw)
    rc, _ = _rc("rope_kv_store", FAKE, 5120, 1, ctypes.addressof(a), None)
    assert rc == code
    rc, _ = _rc("qmv_qkv_rope", 4, FAKE, 2048, FAKE, 2048, 1, ctypes.addressof(a), None)
    assert rc == code


def test_rope_gate_widens_the_stacked_rows():
    # with 32 gate heads the stacked output is (32 + 2 * 8 + 32) * 64 = 5120 wide
    a = _rope(n_gate_heads=32, gate_out=FAKE, ldg=2048)
    rc, msg = _rc("rope_kv_store", FAKE, 3072, 1, ctypes.addressof(a), None)
    assert rc == q4.Q4_EINVAL and "n_gate_heads" in msg
    rc, msg = _rc("qmv_qkv_rope", 4, FAKE, 8192, FAKE, 8192, 1, ctypes.addressof(a), None)
    assert rc == q4.Q4_EUNSUPPORTED and "4096" in msg


def test_rope_struct_layout_matches_header(tmp_path):
    """The ctypes mirror has the C struct's size and field offsets (checked with the host C compiler)."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no host C compiler")
    fields = [f for f, _ in q4.RopeKv._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"q4g64.h\"\nint main(void) {\n"
                   "  printf(\"%zu\\n\", sizeof(q4_rope_kv));\n"
                   + "".join(f"  printf(\"%zu\\n\", offsetof(q4_rope_kv, {f}));\n" for f in fields) + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(q4.RopeKv)
    assert got[1:] == [getattr(q4.RopeKv, f).offset for f in fields]


def test_rope_calls_reject_bad_shapes():
    a = _rope()
    assert _rc("rope_kv_store", FAKE, 3072, 1, None, None)[0] == q4.Q4_EINVAL
    assert _rc("rope_kv_store", FAKE, 3000, 1, ctypes.addressof(a), None)[0] == q4.Q4_EINVAL  # ldqkv < N
    assert _rc("rope_kv_store", FAKE, 3072, 0, ctypes.addressof(a), None)[0] == q4.Q4_EINVAL
    assert _rc("qmv_qkv_rope", 5, FAKE, 2048, FAKE, 2048, 1, ctypes.addressof(a), None)[0] == q4.Q4_EINVAL
    assert _rc("qmv_qkv_rope", 4, FAKE, 2048, FAKE, 2048, 17, ctypes.addressof(a), None)[0] == q4.Q4_EINVAL
    rc, msg = _rc("qmv_qkv_rope", 4, FAKE, 8192, FAKE, 8192, 1, ctypes.addressof(a), None)
    assert rc == q4.Q4_EUNSUPPORTED and "4096" in msg


def test_split_work_bytes_and_rejections():
    f = q4.lib().qmv_split_work_bytes
    # w2 of the decode FFN step (128 column tiles, 32 segments), one float32 row, two shares:
    # 128 counters in a 512-byte block, then 128 tiles x 32 segments x 64 partials
    assert f(4, 2048, 8192, q4.Q4_F32, 1, 2) == 512 + 128 * 32 * 64 * 4
    assert f(4, 2048, 8192, q4.Q4_F32, 1, 0) == f(4, 2048, 8192, q4.Q4_F32, 1, 2)  # automatic: 2 x 128 tiles fill 256 CUs
    assert f(4, 2048, 8192, q4.Q4_BF16, 16, 0) == 512 + 128 * 32 * 4 * 64 * 4  # 16 bf16 rows: 4 row slots per lane group
    for bad in ((5, 2048, 8192, q4.Q4_F32, 1, 0), (4, 100, 8192, q4.Q4_F32, 1, 0), (4, 2048, 8192, 7, 1, 0),
                (4, 2048, 8192, q4.Q4_F32, 17, 0), (4, 2048, 8192, q4.Q4_F32, 1, 17), (4, 2048, 32768, q4.Q4_F32, 1, 0)):
        assert f(*bad) == 0, bad
    base = (4, FAKE, 2048, 8192, FAKE, q4.Q4_F32, 8192, 1, FAKE, 2048)
    assert _rc("qmv_rows_split", *base, 17, FAKE, 1 << 20, None)[0] == q4.Q4_EINVAL
    assert _rc("qmv_rows_split", *base, -1, FAKE, 1 << 20, None)[0] == q4.Q4_EINVAL
    assert _rc("qmv_rows_split", *base, 2, None, 1 << 20, None)[0] == q4.Q4_EALIGN
    assert _rc("qmv_rows_split", *base, 2, FAKE + 16, 1 << 20, None)[0] == q4.Q4_EALIGN
    rc, msg = _rc("qmv_rows_split", *base, 2, FAKE, 1000, None)
    assert rc == q4.Q4_EINVAL and "work_bytes" in msg
    assert _rc("qmv_rows_split", 4, FAKE, 2048, 8192, FAKE, q4.Q4_F32, 8192, 0, FAKE, 2048, 2, FAKE, 1 << 20, None)[0] == q4.Q4_EINVAL
