"""q4g64 on MI355X: Python binding of the C-ABI library ``libq4g64.so``.

Argument marshalling only. Every step of the computation runs in the HIP
kernels behind ``include/q4g64.h``; PyTorch provides device memory and the
stream. If the library is not built, every call raises: there is no fallback.

Tensors: canonical weights are ``wq`` int32/uint32 [N][K/8] (bit patterns),
``scales``/``biases`` int16/uint16/bfloat16 [N][K/64] (bf16 bit patterns);
activations are ``torch.bfloat16`` (or ``torch.float32`` for ``qmv_rows``).
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4g64.so")

Q4_OK, Q4_EINVAL, Q4_EALIGN, Q4_EDEVICE, Q4_EUNSUPPORTED = 0, -1, -2, -3, -4
Q4_BF16, Q4_F32, Q4_BF16X3, Q4_BF16X3T = 0, 1, 2, 3

_lib = None

_I64 = ctypes.c_int64
_P = ctypes.c_void_p
_SIGNATURES = {
    "q4g64_abi_version": (ctypes.c_int, []),
    "q4g64_packed_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "q4g64_x3t_bytes": (ctypes.c_size_t, [_I64, ctypes.c_int]),
    "pack_q4g64": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P, _P]),
    "unpack_q4g64": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P]),
    "qmv_rows": (ctypes.c_int, [_P, _I64, _I64, _P, ctypes.c_int, _I64, ctypes.c_int, _P, _I64, _P]),
    "qmv_w13_swiglu": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, ctypes.c_int, _P, _I64, _P]),
    "qmm_window": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, _I64, _P, ctypes.c_int, _I64, _P]),
    "qmm_cut": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, _P, ctypes.c_int, _P, ctypes.c_int, _I64, _P]),
    "qg64_packed_bytes": (ctypes.c_size_t, [ctypes.c_int, _I64, _I64]),
    "pack_qg64": (ctypes.c_int, [ctypes.c_int, _P, _P, _P, _I64, _I64, _P, _P]),
    "unpack_qg64": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _P, _P, _P, _P]),
    "qmv_rows_qg64": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _P, ctypes.c_int, _I64, ctypes.c_int, _P, _I64, _P]),
    "qmv_w13_swiglu_qg64": (ctypes.c_int, [ctypes.c_int, _P, _P, _I64, _I64, _P, _I64, ctypes.c_int, _P, _I64, _P]),
    "qmv_w13_swiglu_x3": (ctypes.c_int, [ctypes.c_int, _P, _P, _I64, _I64, _P, _I64, ctypes.c_int, _P, _I64, _P]),
    "qmv_w13_swiglu_x3t": (ctypes.c_int, [ctypes.c_int, _P, _P, _I64, _I64, _P, _I64, ctypes.c_int, _P, _P]),
    "qmm_window_qg64": (ctypes.c_int, [ctypes.c_int, _P, _P, _I64, _I64, _P, _I64, _I64, _P, ctypes.c_int, _I64, _P]),
    "qmm_cut_qg64": (ctypes.c_int, [ctypes.c_int, _P, _P, _I64, _I64, _P, _I64, _P, ctypes.c_int, _P, ctypes.c_int, _I64, _P]),
    "fp8b_packed_bytes": (ctypes.c_size_t, [_I64, _I64]),
    "pack_fp8b": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P]),
    "unpack_fp8b": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P]),
    "qmv_rows_fp8b": (ctypes.c_int, [_P, _I64, _I64, _P, ctypes.c_int, _I64, ctypes.c_int, _P, _I64, _P]),
    "qmv_w13_swiglu_fp8b": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, ctypes.c_int, _P, _I64, _P]),
    "qmv_w13_swiglu_x3_fp8b": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, ctypes.c_int, _P, _I64, _P]),
    "qmv_w13_swiglu_x3t_fp8b": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, ctypes.c_int, _P, _P]),
    "qmm_window_fp8b": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, _I64, _P, ctypes.c_int, _I64, _P]),
    "qmm_cut_fp8b": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _I64, _P, ctypes.c_int, _P, ctypes.c_int, _I64, _P]),
    "rope_kv_store": (ctypes.c_int, [_P, _I64, ctypes.c_int, _P, _P]),
    "qmv_qkv_rope": (ctypes.c_int, [ctypes.c_int, _P, _I64, _P, _I64, ctypes.c_int, _P, _P]),
    "qmv_window_costs": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _P, ctypes.c_int, _I64, _P, _I64, ctypes.c_int, _P, _P]),
    "qmv_window_cost": (ctypes.c_float, [_P, ctypes.c_int]),
    "q4g64_ffn_work_bytes": (ctypes.c_size_t, [_I64, _I64, ctypes.c_int]),
    "qmv_split_work_bytes": (ctypes.c_size_t, [ctypes.c_int, _I64, _I64, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "qmv_rows_split": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _P, ctypes.c_int, _I64, ctypes.c_int, _P, _I64, ctypes.c_int,
                                      _P, ctypes.c_size_t, _P]),
    "qmv_split_noalloc_max_bytes": (ctypes.c_size_t, []),
    "qmv_rows_split_noalloc": (ctypes.c_int, [ctypes.c_int, _P, _I64, _I64, _P, ctypes.c_int, _I64, ctypes.c_int, _P, _I64,
                                              ctypes.c_int, _P]),
    "qmv_ffn": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _P, _I64, ctypes.c_int, _P, _I64, _P, _I64, _P, _P]),
    "q4_last_error": (ctypes.c_char_p, []),
}


class Q4Error(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m bit_weight_only_q4g64_amd.build` "
                "(the q4g64 ops have no non-HIP implementation)"
            )
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(fn: str, status: int) -> None:
    if status != Q4_OK:
        raise Q4Error(fn, status, lib().q4_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _rowmajor(t: torch.Tensor, name: str) -> int:
    """Row stride (elements) of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    return t.stride(0)


def _planes_ld(t: torch.Tensor, name: str) -> int:
    """Row stride of a [3][R][ld] bf16 planes tensor (Q4_BF16X3): contiguous rows, plane p at p * R * ld."""
    if t.dim() != 3 or t.shape[0] != 3 or t.dtype != torch.bfloat16 or t.stride(2) != 1 or t.stride(0) != t.shape[1] * t.stride(1):
        raise ValueError(f"{name} must be bfloat16 planes [3][R][ld] with rows of stride ld and planes of stride R * ld")
    return t.stride(1)


class TiledPlanes:
    """R rows of K float32 activations as their three exact bf16 pieces in the
    matvec's fragment order (Q4_BF16X3T), as qmv_w13_swiglu(..., planes="tiled")
    writes them: `data` is a flat bfloat16 tensor of x3t_bytes(K, R) / 2 values."""

    def __init__(self, data: torch.Tensor, rows: int, k: int):
        if data.dtype != torch.bfloat16 or not data.is_contiguous() or data.numel() * 2 < x3t_bytes(k, rows):
            raise ValueError("data must be a contiguous bfloat16 tensor of at least x3t_bytes(K, R) bytes")
        self.data, self.rows, self.k = data, rows, k

    @staticmethod
    def empty(rows: int, k: int, device) -> "TiledPlanes":
        n = x3t_bytes(k, rows)
        if n == 0:
            raise ValueError(f"no fragment-ordered planes for K={k}, R={rows}")
        return TiledPlanes(torch.empty(n // 2, dtype=torch.bfloat16, device=device), rows, k)


def x3t_bytes(K: int, R: int) -> int:
    """Bytes of R rows of K activations as Q4_BF16X3T (0 if invalid)."""
    return int(lib().q4g64_x3t_bytes(K, R))


def _x_ptr(x) -> int:
    return x.data.data_ptr() if isinstance(x, TiledPlanes) else x.data_ptr()


def _x_arg(x):
    """(x_dtype, ldx, R) of decode activations: bf16 or float32 rows [R][ldx], the three bf16 planes of float32
    rows [3][R][ldx] (Q4_BF16X3, as qmv_w13_swiglu(..., planes=True) writes them), or TiledPlanes (Q4_BF16X3T)."""
    if isinstance(x, TiledPlanes):
        return Q4_BF16X3T, x.k, x.rows
    if x.dim() == 3:
        return Q4_BF16X3, _planes_ld(x, "x"), x.shape[1]
    if x.dtype == torch.bfloat16:
        return Q4_BF16, _rowmajor(x, "x"), x.shape[0]
    if x.dtype == torch.float32:
        return Q4_F32, _rowmajor(x, "x"), x.shape[0]
    raise ValueError("x must be bfloat16 or float32 rows, or bfloat16 planes [3][R][ld]")


def packed_bytes(N: int, K: int, bits: int = 4) -> int:
    if bits == 4:
        return int(lib().q4g64_packed_bytes(N, K))
    return int(lib().qg64_packed_bytes(bits, N, K))


def pack(wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, bits: int = 4) -> torch.Tensor:
    """Canonical MLX group-64 weights of 4, 6 or 8 bits (device tensors) ->
    packed device layout (uint8 tensor). wq is [N][K*bits/32] words."""
    for t, name in ((wq, "wq"), (scales, "scales"), (biases, "biases")):
        _dev(t, name)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    N, K = wq.shape[0], wq.shape[1] * 32 // bits
    if wq.element_size() != 4 or scales.element_size() != 2 or biases.element_size() != 2:
        raise ValueError("wq holds 32-bit words, scales/biases 16-bit bf16 patterns")
    if tuple(scales.shape) != (N, K // 64) or tuple(biases.shape) != (N, K // 64):
        raise ValueError("scales and biases must be [N][K/64]")
    nbytes = packed_bytes(N, K, bits)
    if nbytes == 0:
        raise Q4Error("pack_qg64", Q4_EINVAL, f"invalid shape N={N} K={K} bits={bits}")
    out = torch.empty(nbytes, dtype=torch.uint8, device=wq.device)
    if bits == 4:
        _check("pack_q4g64", lib().pack_q4g64(wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), N, K, out.data_ptr(), _stream()))
    else:
        _check("pack_qg64",
               lib().pack_qg64(bits, wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), N, K, out.data_ptr(), _stream()))
    return out


def unpack(packed: torch.Tensor, N: int, K: int, bits: int = 4):
    """Packed layout -> canonical (wq int32 [N][K*bits/32], scales int16, biases int16 [N][K/64])."""
    _dev(packed, "packed")
    wq = torch.empty((N, K * bits // 32), dtype=torch.int32, device=packed.device)
    sc = torch.empty((N, K // 64), dtype=torch.int16, device=packed.device)
    bi = torch.empty((N, K // 64), dtype=torch.int16, device=packed.device)
    if bits == 4:
        _check("unpack_q4g64", lib().unpack_q4g64(packed.data_ptr(), N, K, wq.data_ptr(), sc.data_ptr(), bi.data_ptr(), _stream()))
    else:
        _check("unpack_qg64",
               lib().unpack_qg64(bits, packed.data_ptr(), N, K, wq.data_ptr(), sc.data_ptr(), bi.data_ptr(), _stream()))
    return wq, sc, bi


def qmv_rows(packed: torch.Tensor, N: int, K: int, x: torch.Tensor, y: torch.Tensor | None = None, bits: int = 4) -> torch.Tensor:
    """y[r] = W x[r] for the R (1..16) rows of x (bf16 or float32 [R][ld], float32 as bf16 planes [3][R][ld], or
    TiledPlanes); W has 4-, 6- or 8-bit codes."""
    _dev(packed, "packed")
    _dev(x.data if isinstance(x, TiledPlanes) else x, "x")
    xd, ldx, R = _x_arg(x)
    dev = x.data.device if isinstance(x, TiledPlanes) else x.device
    if y is None:
        y = torch.empty((R, N), dtype=torch.float32, device=dev)
    if y.dtype != torch.float32 or y.shape[0] < R:
        raise ValueError("y must be float32 with at least R rows")
    if bits == 4:
        _check("qmv_rows", lib().qmv_rows(packed.data_ptr(), N, K, _x_ptr(x), xd, ldx, R, y.data_ptr(), _rowmajor(y, "y"), _stream()))
    else:
        _check("qmv_rows_qg64",
               lib().qmv_rows_qg64(bits, packed.data_ptr(), N, K, _x_ptr(x), xd, ldx, R, y.data_ptr(), _rowmajor(y, "y"), _stream()))
    return y


def split_work_bytes(N: int, K: int, x_dtype: int, R: int, splits: int = 0, bits: int = 4) -> int:
    """Workspace bytes qmv_rows_split needs for this shape (0: invalid arguments)."""
    return int(lib().qmv_split_work_bytes(bits, N, K, x_dtype, R, splits))


def split_workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled, 256-byte aligned device workspace for qmv_rows_split (torch's allocations are)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def qmv_rows_split(packed: torch.Tensor, N: int, K: int, x: torch.Tensor, work: torch.Tensor, y: torch.Tensor | None = None,
                   splits: int = 0, bits: int = 4) -> torch.Tensor:
    """qmv_rows with K split over several workgroups per column tile (bit-identical to qmv_rows); ``work`` is a
    workspace from split_workspace() of at least split_work_bytes() bytes, not shared by concurrent calls."""
    _dev(packed, "packed")
    _dev(x.data if isinstance(x, TiledPlanes) else x, "x")
    _dev(work, "work")
    xd, ldx, R = _x_arg(x)
    dev = x.data.device if isinstance(x, TiledPlanes) else x.device
    if y is None:
        y = torch.empty((R, N), dtype=torch.float32, device=dev)
    if y.dtype != torch.float32 or y.shape[0] < R:
        raise ValueError("y must be float32 with at least R rows")
    _check("qmv_rows_split", lib().qmv_rows_split(bits, packed.data_ptr(), N, K, _x_ptr(x), xd, ldx, R, y.data_ptr(),
                                                  _rowmajor(y, "y"), splits, work.data_ptr(), work.numel(), _stream()))
    return y


def qmv_w13_swiglu(p1: torch.Tensor, p3: torch.Tensor, N: int, K: int, x: torch.Tensor, y: torch.Tensor | None = None,
                   bits: int = 4, planes=False):
    """y[r] = silu(W1 x[r]) * (W3 x[r]) for the 1..16 bf16 rows of x; W1, W3 have 4-, 6- or 8-bit codes.
    planes=True: y is written as the three exact bf16 pieces of each float32 result, planes [3][R][N];
    planes="tiled": the same pieces in fragment order (returns TiledPlanes)."""
    _dev(p1, "packed_w1")
    _dev(p3, "packed_w3")
    _dev(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    R = x.shape[0]
    if planes == "tiled":
        if y is None:
            y = TiledPlanes.empty(R, N, x.device)
        _check("qmv_w13_swiglu_x3t", lib().qmv_w13_swiglu_x3t(bits, p1.data_ptr(), p3.data_ptr(), N, K, x.data_ptr(), _rowmajor(x, "x"),
                                                              R, y.data.data_ptr(), _stream()))
        return y
    if planes:
        if y is None:
            y = torch.empty((3, R, N), dtype=torch.bfloat16, device=x.device)
        _check("qmv_w13_swiglu_x3", lib().qmv_w13_swiglu_x3(bits, p1.data_ptr(), p3.data_ptr(), N, K, x.data_ptr(), _rowmajor(x, "x"), R,
                                                            y.data_ptr(), _planes_ld(y, "y"), _stream()))
        return y
    if y is None:
        y = torch.empty((R, N), dtype=torch.float32, device=x.device)
    if bits == 4:
        _check(
            "qmv_w13_swiglu",
            lib().qmv_w13_swiglu(p1.data_ptr(), p3.data_ptr(), N, K, x.data_ptr(), _rowmajor(x, "x"), R, y.data_ptr(), _rowmajor(y, "y"),
                                 _stream()),
        )
    else:
        _check(
            "qmv_w13_swiglu_qg64",
            lib().qmv_w13_swiglu_qg64(bits, p1.data_ptr(), p3.data_ptr(), N, K, x.data_ptr(), _rowmajor(x, "x"), R, y.data_ptr(),
                                      _rowmajor(y, "y"), _stream()),
        )
    return y


def _out_dtype(dtype) -> int:
    if dtype == torch.float32:
        return Q4_F32
    if dtype == torch.bfloat16:
        return Q4_BF16
    raise ValueError("output dtype must be float32 or bfloat16")


def qmm_window(pa: torch.Tensor, pb: torch.Tensor | None, N: int, K: int, x: torch.Tensor, y: torch.Tensor | None = None,
               out_dtype=torch.float32, bits: int = 4) -> torch.Tensor:
    """Prompt window: y = A x (pb None) or silu(A x) * (B x), for all M rows of x; 4-, 6- or 8-bit codes."""
    _dev(pa, "packed_a")
    _dev(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    pbp = None if pb is None else pb.data_ptr()
    if bits == 4:
        _check("qmm_window", lib().qmm_window(pa.data_ptr(), pbp, N, K, x.data_ptr(), _rowmajor(x, "x"), M, y.data_ptr(),
                                              _out_dtype(y.dtype), _rowmajor(y, "y"), _stream()))
    else:
        _check("qmm_window_qg64", lib().qmm_window_qg64(bits, pa.data_ptr(), pbp, N, K, x.data_ptr(), _rowmajor(x, "x"), M,
                                                        y.data_ptr(), _out_dtype(y.dtype), _rowmajor(y, "y"), _stream()))
    return y


def qmm_cut(pa: torch.Tensor, pb: torch.Tensor | None, N: int, K: int, x: torch.Tensor, windows, y: torch.Tensor | None = None,
            out_dtype=torch.float32, bits: int = 4) -> torch.Tensor:
    """Run the prompt x through consecutive windows of the given row counts."""
    _dev(pa, "packed_a")
    _dev(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    windows = [int(w) for w in windows]
    if sum(windows) != x.shape[0]:
        raise ValueError("window row counts must add up to the prompt's rows")
    if y is None:
        y = torch.empty((x.shape[0], N), dtype=out_dtype, device=x.device)
    arr = (ctypes.c_int64 * len(windows))(*windows)
    pbp = None if pb is None else pb.data_ptr()
    if bits == 4:
        _check("qmm_cut", lib().qmm_cut(pa.data_ptr(), pbp, N, K, x.data_ptr(), _rowmajor(x, "x"), arr, len(windows), y.data_ptr(),
                                        _out_dtype(y.dtype), _rowmajor(y, "y"), _stream()))
    else:
        _check("qmm_cut_qg64", lib().qmm_cut_qg64(bits, pa.data_ptr(), pbp, N, K, x.data_ptr(), _rowmajor(x, "x"), arr,
                                                  len(windows), y.data_ptr(), _out_dtype(y.dtype), _rowmajor(y, "y"), _stream()))
    return y


# The qmv_ffn workspace (byte offsets of 32-bit words): the error word (1 once
# a wait of the one-launch step gave up) and that step's call counter.
FFN_ERR_OFFSET = 18 * 128
FFN_FLOW_EPOCH_OFFSET = 4096


def ffn_work_bytes(N1: int, N2: int, R: int) -> int:
    return int(lib().q4g64_ffn_work_bytes(N1, N2, R))


def ffn_workspace(N1: int, N2: int, R: int, device="cuda") -> torch.Tensor:
    """A zeroed workspace for qmv_ffn calls (any row count; reusable by later calls on the same stream)."""
    nbytes = ffn_work_bytes(N1, N2, R)
    if nbytes == 0:
        raise Q4Error("q4g64_ffn_work_bytes", Q4_EINVAL, f"invalid N1={N1} N2={N2} R={R}")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def ffn_error(work: torch.Tensor) -> int:
    """The workspace's error word (1 if a workgroup of the one-launch step gave up waiting)."""
    return int(work[FFN_ERR_OFFSET : FFN_ERR_OFFSET + 4].view(torch.int32).item())


def qmv_ffn(p1: torch.Tensor, p3: torch.Tensor, p2: torch.Tensor, N1: int, K1: int, N2: int, x: torch.Tensor, work: torch.Tensor,
            z: torch.Tensor | None = None, y: torch.Tensor | None = None):
    """Decode FFN step: z = silu(W1 x) * (W3 x), y = W2 z (float32), for the 1..16 bf16 rows of x (one launch up to 2 rows, two from 3)."""
    for t, name in ((p1, "packed_w1"), (p3, "packed_w3"), (p2, "packed_w2"), (x, "x"), (work, "work")):
        _dev(t, name)
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    R = x.shape[0]
    if work.numel() < ffn_work_bytes(N1, N2, R):
        raise ValueError("work is smaller than ffn_work_bytes(N1, N2, R)")
    if z is None:
        z = torch.empty((R, N1), dtype=torch.float32, device=x.device)
    if y is None:
        y = torch.empty((R, N2), dtype=torch.float32, device=x.device)
    _check(
        "qmv_ffn",
        lib().qmv_ffn(p1.data_ptr(), p3.data_ptr(), p2.data_ptr(), N1, K1, N2, x.data_ptr(), _rowmajor(x, "x"), R, z.data_ptr(),
                      _rowmajor(z, "z"), y.data_ptr(), _rowmajor(y, "y"), work.data_ptr(), _stream()),
    )
    return z, y


WINDOW_COST_ROWS = (1, 2, 4, 8, 16)


def window_costs(packed: torch.Tensor, N: int, K: int, x: torch.Tensor, bits: int = 4, reps: int = 20,
                 y: torch.Tensor | None = None) -> list:
    """Average qmv_rows time (us) at R = 1, 2, 4, 8, 16, measured on the 16 rows of x (a load-time call)."""
    _dev(packed, "packed")
    _dev(x, "x")
    if x.shape[0] < 16:
        raise ValueError("x must hold 16 rows")
    xd = Q4_BF16 if x.dtype == torch.bfloat16 else Q4_F32 if x.dtype == torch.float32 else None
    if xd is None:
        raise ValueError("x must be bfloat16 or float32")
    if y is None:
        y = torch.empty((16, N), dtype=torch.float32, device=x.device)
    out = (ctypes.c_float * 5)()
    _check("qmv_window_costs", lib().qmv_window_costs(bits, packed.data_ptr(), N, K, x.data_ptr(), xd, _rowmajor(x, "x"), y.data_ptr(),
                                                      _rowmajor(y, "y"), reps, ctypes.addressof(out), _stream()))
    return list(out)


def window_cost(costs, R: int) -> float:
    """Interpolated cost of R rows (1..16) from a window_costs table."""
    arr = (ctypes.c_float * 5)(*[float(c) for c in costs])
    return float(lib().qmv_window_cost(ctypes.addressof(arr), R))


# ---- block FP8 (E4M3 bytes, float32 scale per 128 x 128 block) -------------


def fp8b_packed_bytes(N: int, K: int) -> int:
    return int(lib().fp8b_packed_bytes(N, K))


def pack_fp8b(w8: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """E4M3 bytes [N][K] (uint8) and float32 block scales [ceil(N/128)][ceil(K/128)] -> packed layout."""
    for t, name in ((w8, "w8"), (scales, "scales")):
        _dev(t, name)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if w8.dtype != torch.uint8 or scales.dtype != torch.float32:
        raise ValueError("w8 is uint8 and scales float32")
    N, K = w8.shape
    if tuple(scales.shape) != (-(-N // 128), -(-K // 128)):
        raise ValueError("scales must be [ceil(N/128)][ceil(K/128)]")
    nbytes = fp8b_packed_bytes(N, K)
    if nbytes == 0:
        raise Q4Error("pack_fp8b", Q4_EINVAL, f"invalid shape N={N} K={K}")
    out = torch.empty(nbytes, dtype=torch.uint8, device=w8.device)
    _check("pack_fp8b", lib().pack_fp8b(w8.data_ptr(), scales.data_ptr(), N, K, out.data_ptr(), _stream()))
    return out


def unpack_fp8b(packed: torch.Tensor, N: int, K: int):
    """Packed layout -> (w8 uint8 [N][K], scales float32 [ceil(N/128)][ceil(K/128)])."""
    _dev(packed, "packed")
    w8 = torch.empty((N, K), dtype=torch.uint8, device=packed.device)
    sc = torch.empty((-(-N // 128), -(-K // 128)), dtype=torch.float32, device=packed.device)
    _check("unpack_fp8b", lib().unpack_fp8b(packed.data_ptr(), N, K, w8.data_ptr(), sc.data_ptr(), _stream()))
    return w8, sc


def qmv_rows_fp8b(packed: torch.Tensor, N: int, K: int, x, y: torch.Tensor | None = None) -> torch.Tensor:
    """y[r] = W x[r] for the 1..16 rows of x (as qmv_rows), W block FP8."""
    _dev(packed, "packed")
    _dev(x.data if isinstance(x, TiledPlanes) else x, "x")
    xd, ldx, R = _x_arg(x)
    if y is None:
        y = torch.empty((R, N), dtype=torch.float32, device=x.data.device if isinstance(x, TiledPlanes) else x.device)
    _check("qmv_rows_fp8b", lib().qmv_rows_fp8b(packed.data_ptr(), N, K, _x_ptr(x), xd, ldx, R, y.data_ptr(),
                                                _rowmajor(y, "y"), _stream()))
    return y


def qmv_w13_swiglu_fp8b(p1: torch.Tensor, p3: torch.Tensor, N: int, K: int, x: torch.Tensor, y: torch.Tensor | None = None,
                        planes=False):
    """y[r] = silu(W1 x[r]) * (W3 x[r]) for the 1..16 bf16 rows of x, W1 and W3 block FP8 (planes: as qmv_w13_swiglu)."""
    _dev(p1, "packed_w1")
    _dev(p3, "packed_w3")
    _dev(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    R = x.shape[0]
    if planes == "tiled":
        if y is None:
            y = TiledPlanes.empty(R, N, x.device)
        _check("qmv_w13_swiglu_x3t_fp8b", lib().qmv_w13_swiglu_x3t_fp8b(p1.data_ptr(), p3.data_ptr(), N, K, x.data_ptr(),
                                                                        _rowmajor(x, "x"), R, y.data.data_ptr(), _stream()))
        return y
    if planes:
        if y is None:
            y = torch.empty((3, R, N), dtype=torch.bfloat16, device=x.device)
        _check("qmv_w13_swiglu_x3_fp8b", lib().qmv_w13_swiglu_x3_fp8b(p1.data_ptr(), p3.data_ptr(), N, K, x.data_ptr(), _rowmajor(x, "x"),
                                                                      R, y.data_ptr(), _planes_ld(y, "y"), _stream()))
        return y
    if y is None:
        y = torch.empty((R, N), dtype=torch.float32, device=x.device)
    _check("qmv_w13_swiglu_fp8b", lib().qmv_w13_swiglu_fp8b(p1.data_ptr(), p3.data_ptr(), N, K, x.data_ptr(), _rowmajor(x, "x"), R,
                                                            y.data_ptr(), _rowmajor(y, "y"), _stream()))
    return y


def qmm_window_fp8b(pa: torch.Tensor, pb: torch.Tensor | None, N: int, K: int, x: torch.Tensor, y: torch.Tensor | None = None,
                    out_dtype=torch.float32) -> torch.Tensor:
    """Prompt window with block-FP8 weights: y = A x or silu(A x) * (B x)."""
    _dev(pa, "packed_a")
    _dev(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    _check("qmm_window_fp8b", lib().qmm_window_fp8b(pa.data_ptr(), None if pb is None else pb.data_ptr(), N, K, x.data_ptr(),
                                                    _rowmajor(x, "x"), M, y.data_ptr(), _out_dtype(y.dtype), _rowmajor(y, "y"), _stream()))
    return y


def qmm_cut_fp8b(pa: torch.Tensor, pb: torch.Tensor | None, N: int, K: int, x: torch.Tensor, windows, y: torch.Tensor | None = None,
                 out_dtype=torch.float32) -> torch.Tensor:
    """The prompt x through consecutive windows, block-FP8 weights."""
    _dev(pa, "packed_a")
    _dev(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    windows = [int(w) for w in windows]
    if sum(windows) != x.shape[0]:
        raise ValueError("window row counts must add up to the prompt's rows")
    if y is None:
        y = torch.empty((x.shape[0], N), dtype=out_dtype, device=x.device)
    arr = (ctypes.c_int64 * len(windows))(*windows)
    _check("qmm_cut_fp8b", lib().qmm_cut_fp8b(pa.data_ptr(), None if pb is None else pb.data_ptr(), N, K, x.data_ptr(),
                                              _rowmajor(x, "x"), arr, len(windows), y.data_ptr(), _out_dtype(y.dtype), _rowmajor(y, "y"),
                                              _stream()))
    return y


# ---- attention-side decode epilogue: QK norm, partial RoPE, KV store -------


class RopeKv(ctypes.Structure):
    """Mirror of the C struct q4_rope_kv (device pointers as integers)."""

    _fields_ = [("pos", ctypes.c_void_p), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("rot_dims", ctypes.c_int32), ("theta", ctypes.c_float), ("gamma_q", ctypes.c_void_p),
                ("gamma_k", ctypes.c_void_p), ("eps", ctypes.c_float), ("q_out", ctypes.c_void_p), ("ldq", ctypes.c_int64),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("cache_dtype", ctypes.c_int32),
                ("ring_len", ctypes.c_int64), ("n_gate_heads", ctypes.c_int32), ("gate_out", ctypes.c_void_p),
                ("ldg", ctypes.c_int64), ("cache_row_stride", ctypes.c_int64)]


def _rope_args(pos, n_q, n_kv, rot, theta, q_out, k_cache, v_cache, gamma_q, gamma_k, eps, gate_out=None):
    for t, name in ((pos, "pos"), (q_out, "q_out"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, name)
    n_gate, gate_ptr, ldg = 0, None, 0
    if gate_out is not None:
        _dev(gate_out, "gate_out")
        if gate_out.dtype != torch.float32 or gate_out.dim() != 2 or gate_out.shape[1] % 64:
            raise ValueError("gate_out is a float32 [R][n_gate_heads * 64] tensor")
        n_gate, gate_ptr, ldg = gate_out.shape[1] // 64, gate_out.data_ptr(), _rowmajor(gate_out, "gate_out")
    if pos.dtype != torch.int32 or q_out.dtype != torch.float32:
        raise ValueError("pos is int32 and q_out float32")
    if k_cache.dtype != v_cache.dtype or k_cache.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("the caches are both float32 or both bfloat16")
    if tuple(k_cache.shape[-2:]) != (n_kv, 64) or k_cache.dim() not in (3, 4) or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or not k_cache.is_contiguous() or not v_cache.is_contiguous():
        raise ValueError("the caches are contiguous [ring][n_kv_heads][64] (one ring for every row) or "
                         "[rows][ring][n_kv_heads][64] (a ring per row)")
    if k_cache.dim() == 4 and k_cache.shape[0] < pos.numel():
        raise ValueError("a per-row cache needs a ring for every row")
    ring = k_cache.shape[-3]
    row_stride = ring * n_kv * 64 if k_cache.dim() == 4 else 0
    for g, name in ((gamma_q, "gamma_q"), (gamma_k, "gamma_k")):
        if g is not None:
            _dev(g, name)
            if g.dtype != torch.float32 or g.numel() != 64:
                raise ValueError(f"{name} is a float32 [64] vector")
    return RopeKv(pos.data_ptr(), n_q, n_kv, rot, theta, None if gamma_q is None else gamma_q.data_ptr(),
                  None if gamma_k is None else gamma_k.data_ptr(), eps, q_out.data_ptr(), _rowmajor(q_out, "q_out"),
                  k_cache.data_ptr(), v_cache.data_ptr(), Q4_F32 if k_cache.dtype == torch.float32 else Q4_BF16, ring,
                  n_gate, gate_ptr, ldg, row_stride)


def rope_kv_store(qkv: torch.Tensor, pos: torch.Tensor, n_q: int, n_kv: int, rot: int, theta: float, q_out: torch.Tensor,
                  k_cache: torch.Tensor, v_cache: torch.Tensor, gamma_q=None, gamma_k=None, eps: float = 1e-6,
                  gate_out=None) -> None:
    """QK norm (when gammas are given), partial RoPE and the KV store on a float32 q/k/v output
    [R][(n_q+2n_kv)*64]; with ``gate_out`` [R][n_gate*64], the gate heads that follow v are copied there."""
    _dev(qkv, "qkv")
    if qkv.dtype != torch.float32:
        raise ValueError("qkv must be float32")
    a = _rope_args(pos, n_q, n_kv, rot, theta, q_out, k_cache, v_cache, gamma_q, gamma_k, eps, gate_out)
    _check("rope_kv_store", lib().rope_kv_store(qkv.data_ptr(), _rowmajor(qkv, "qkv"), qkv.shape[0], ctypes.addressof(a), _stream()))


def qmv_qkv_rope(packed: torch.Tensor, K: int, x: torch.Tensor, pos: torch.Tensor, n_q: int, n_kv: int, rot: int, theta: float,
                 q_out: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, gamma_q=None, gamma_k=None, eps: float = 1e-6,
                 bits: int = 4, gate_out=None) -> None:
    """The stacked q/k/v(/gate) decode matvec with QK norm, partial RoPE and the KV store in one launch
    (1..16 bf16 rows); ``gate_out`` [R][n_gate*64] receives the gate heads stacked after v."""
    _dev(packed, "packed_qkv")
    _dev(x, "x")
    if x.dtype != torch.bfloat16:
        raise ValueError("x must be bfloat16")
    a = _rope_args(pos, n_q, n_kv, rot, theta, q_out, k_cache, v_cache, gamma_q, gamma_k, eps, gate_out)
    _check("qmv_qkv_rope", lib().qmv_qkv_rope(bits, packed.data_ptr(), K, x.data_ptr(), _rowmajor(x, "x"), x.shape[0],
                                              ctypes.addressof(a), _stream()))
