"""The three-plane handoff of float32 activations (Q4_BF16X3): the fused
SwiGLU can write each float32 result as its three exact bf16 pieces, and the
decode matvec takes such planes in place of float32 rows.

* The planes written by qmv_w13_swiglu(..., planes=True) are, bit for bit,
  the truncation split of the float32 results of the same call without
  planes (the split is computed here on the host), and the pieces add up to
  the float32 value exactly.
* qmv_rows on planes split on the host equals qmv_rows on the float32 rows
  bit for bit, at row counts whose activations are staged in LDS and at
  row counts where they are read from memory, for every code format.
* The decode FFN step through planes equals the step through float32."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import synthetic
from tests.gpu_helpers import DEV, bits32, dev_bf16, dev_weight, say

pytestmark = pytest.mark.gpu

FORMATS = (4, 6, 8, "fp8")


def split_planes(z: np.ndarray):
    """Q4_BF16X3 encoding of float32 values: h = top 16 bits of z, m = top 16 bits of z - h, l = z - h - m."""
    z = np.ascontiguousarray(z, dtype=np.float32)
    hu = z.view(np.uint32) & np.uint32(0xFFFF0000)
    r1 = z - hu.view(np.float32)
    mu = r1.view(np.uint32) & np.uint32(0xFFFF0000)
    r2 = r1 - mu.view(np.float32)
    assert np.all((r2.view(np.uint32) & np.uint32(0xFFFF)) == 0)  # l is exact in bf16
    return np.stack([(hu >> 16).astype(np.uint16), (mu >> 16).astype(np.uint16), (r2.view(np.uint32) >> 16).astype(np.uint16)])


def planes_to_f64(p: np.ndarray) -> np.ndarray:
    f = (p.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return (f[0] + f[1]) + f[2]


def _weight(rng, fmt, name, N, K):
    if fmt == "fp8":
        w = synthetic.draw_fp8_weight(rng, name, N, K)
        return q4.pack_fp8b(torch.from_numpy(np.ascontiguousarray(w.w8)).to(DEV), torch.from_numpy(np.ascontiguousarray(w.scales)).to(DEV))
    return dev_weight(synthetic.draw_qweight(rng, name, N, K, bits=fmt))


def _w13(p1, p3, fmt, N, K, x, planes):
    if fmt == "fp8":
        return q4.qmv_w13_swiglu_fp8b(p1, p3, N, K, x, planes=planes)
    return q4.qmv_w13_swiglu(p1, p3, N, K, x, bits=fmt, planes=planes)


def _rows(p, fmt, N, K, x):
    if fmt == "fp8":
        return q4.qmv_rows_fp8b(p, N, K, x)
    return q4.qmv_rows(p, N, K, x, bits=fmt)


@pytest.fixture(scope="module")
def ffn():
    rng = np.random.default_rng(960)
    d = {}
    for fmt in FORMATS:
        d[fmt] = (_weight(rng, fmt, "w1", 1024, 2048), _weight(rng, fmt, "w3", 1024, 2048), _weight(rng, fmt, "w2", 2048, 1024))
    d["x"] = dev_bf16(synthetic.draw_bf16_rows(rng, 16, 2048))
    return d


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("R", [1, 5, 16])
def test_w13_planes_are_the_exact_split(ffn, fmt, R):
    say(f"w13 planes fmt={fmt} R={R}")
    p1, p3, _ = ffn[fmt]
    z32 = _w13(p1, p3, fmt, 1024, 2048, ffn["x"][:R], planes=False)
    z3 = _w13(p1, p3, fmt, 1024, 2048, ffn["x"][:R], planes=True)
    torch.cuda.synchronize()
    zh = z32.cpu().numpy()
    got = z3.view(torch.int16).cpu().numpy().view(np.uint16)
    assert got.shape == (3, R, 1024)
    assert np.array_equal(got, split_planes(zh))
    assert np.array_equal(planes_to_f64(got), zh.astype(np.float64))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("R", [1, 3, 4, 7, 16])
def test_rows_on_planes_equal_rows_on_float32(fmt, R):
    """K = 8192: three planes of up to 3 rows fit in LDS; from 4 rows on the fragments come from memory."""
    say(f"qmv_rows planes vs float32 fmt={fmt} R={R}")
    rng = np.random.default_rng(961 + R)
    N, K = 2048, 8192
    p = _weight(rng, fmt, "w2", N, K)
    xf = synthetic.draw_f32_rows(rng, R, K, sigma=0.05)
    x32 = torch.from_numpy(xf).to(DEV)
    x3 = torch.from_numpy(split_planes(xf).view(np.int16)).to(DEV).view(torch.bfloat16)
    y32 = _rows(p, fmt, N, K, x32)
    y3 = _rows(p, fmt, N, K, x3)
    torch.cuda.synchronize()
    assert np.array_equal(bits32(y3), bits32(y32))


def test_rows_on_padded_planes(ffn):
    """Planes with a row stride above K (and the plane stride R * ld that goes with it)."""
    rng = np.random.default_rng(962)
    N, K, R, ld = 512, 1088, 6, 1088 + 24
    p = _weight(rng, 4, "w", N, K)
    xf = synthetic.draw_f32_rows(rng, R, K, sigma=0.3)
    pl = np.zeros((3, R, ld), dtype=np.uint16)
    pl[:, :, :K] = split_planes(xf)
    x3 = torch.from_numpy(pl.view(np.int16)).to(DEV).view(torch.bfloat16)[:, :, :K]
    y3 = q4.qmv_rows(p, N, K, x3)
    y32 = q4.qmv_rows(p, N, K, torch.from_numpy(xf).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(bits32(y3), bits32(y32))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("R", [1, 4, 16])
def test_ffn_step_through_planes(ffn, fmt, R):
    p1, p3, p2 = ffn[fmt]
    x = ffn["x"][:R]
    y32 = _rows(p2, fmt, 2048, 1024, _w13(p1, p3, fmt, 1024, 2048, x, planes=False))
    y3 = _rows(p2, fmt, 2048, 1024, _w13(p1, p3, fmt, 1024, 2048, x, planes=True))
    torch.cuda.synchronize()
    assert np.array_equal(bits32(y3), bits32(y32))


# ---- the same pieces in fragment order (Q4_BF16X3T) -------------------------


def tile_planes(pl: np.ndarray, fill: int = 0) -> np.ndarray:
    """[3][R][K] uint16 planes -> Q4_BF16X3T, written from the layout's definition: piece p of element k of row r at
    ((((k/64) * T + r/4) * 2 + (k/32)%2) * 64 + 4*(r%4) + p + 16*((k/8)%4)) * 8 + k%8, T = 1, 2, 4 tiles for
    R <= 4, 8, 16. Unused slots get `fill`."""
    _, R, K = pl.shape
    T = 1 if R <= 4 else (2 if R <= 8 else 4)
    out = np.full((K // 64) * T * 1024, fill, dtype=np.uint16)
    k = np.arange(K)
    for r in range(R):
        for p in range(3):
            pos = ((((k // 64) * T + r // 4) * 2 + (k // 32) % 2) * 64 + 4 * (r % 4) + p + 16 * ((k // 8) % 4)) * 8 + k % 8
            out[pos] = pl[p, r]
    return out


def used_slots(R: int, K: int) -> np.ndarray:
    return tile_planes(np.ones((3, R, K), dtype=np.uint16), fill=0).astype(bool)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("R", [1, 4, 5, 9, 16])
def test_w13_tiled_planes_are_the_exact_split(ffn, fmt, R):
    say(f"w13 tiled planes fmt={fmt} R={R}")
    p1, p3, _ = ffn[fmt]
    z32 = _w13(p1, p3, fmt, 1024, 2048, ffn["x"][:R], planes=False)
    zt = _w13(p1, p3, fmt, 1024, 2048, ffn["x"][:R], planes="tiled")
    torch.cuda.synchronize()
    assert isinstance(zt, q4.TiledPlanes) and zt.rows == R and zt.k == 1024
    got = zt.data.view(torch.int16).cpu().numpy().view(np.uint16)
    want = tile_planes(split_planes(z32.cpu().numpy()))
    used = used_slots(R, 1024)
    assert got.size == want.size == q4.x3t_bytes(1024, R) // 2
    assert np.array_equal(got[used], want[used])


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("R", [1, 3, 4, 7, 8, 9, 16])
def test_rows_on_tiled_planes_equal_rows_on_float32(fmt, R):
    """K = 8192; the slots the layout leaves unread hold NaN patterns, which must not reach any result."""
    say(f"qmv_rows tiled planes vs float32 fmt={fmt} R={R}")
    rng = np.random.default_rng(971 + R)
    N, K = 2048, 8192
    p = _weight(rng, fmt, "w2", N, K)
    xf = synthetic.draw_f32_rows(rng, R, K, sigma=0.05)
    xt = tile_planes(split_planes(xf), fill=0x7FC1)
    x3t = q4.TiledPlanes(torch.from_numpy(xt.view(np.int16)).to(DEV).view(torch.bfloat16), R, K)
    y32 = _rows(p, fmt, N, K, torch.from_numpy(xf).to(DEV))
    yt = _rows(p, fmt, N, K, x3t)
    torch.cuda.synchronize()
    assert np.array_equal(bits32(yt), bits32(y32))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("R", [1, 4, 16])
def test_ffn_step_through_tiled_planes(ffn, fmt, R):
    p1, p3, p2 = ffn[fmt]
    x = ffn["x"][:R]
    y32 = _rows(p2, fmt, 2048, 1024, _w13(p1, p3, fmt, 1024, 2048, x, planes=False))
    yt = _rows(p2, fmt, 2048, 1024, _w13(p1, p3, fmt, 1024, 2048, x, planes="tiled"))
    torch.cuda.synchronize()
    assert np.array_equal(bits32(yt), bits32(y32))


@pytest.mark.parametrize("N", [64, 512, 8192])
@pytest.mark.parametrize("R", [5, 12, 16])
def test_row_tile_split_keeps_the_bits(N, R):
    """Float32 rows read from memory spread their row tiles over more workgroups while the column tiles leave CUs
    idle (N = 64: 4 column tiles, each row tile its own workgroup; N = 8192: no split). Every float32 form gives
    the same bits, and every row equals its one-row call."""
    say(f"row-tile split N={N} R={R}")
    rng = np.random.default_rng(990 + N + R)
    K = 8192
    p = _weight(rng, 4, "w", N, K)
    xf = synthetic.draw_f32_rows(rng, R, K, sigma=0.2)
    x32 = torch.from_numpy(xf).to(DEV)
    pl = split_planes(xf)
    x3 = torch.from_numpy(pl.view(np.int16)).to(DEV).view(torch.bfloat16)
    xt = q4.TiledPlanes(torch.from_numpy(tile_planes(pl).view(np.int16)).to(DEV).view(torch.bfloat16), R, K)
    y32, y3, yt = (q4.qmv_rows(p, N, K, x) for x in (x32, x3, xt))
    torch.cuda.synchronize()
    assert np.array_equal(bits32(y3), bits32(y32))
    assert np.array_equal(bits32(yt), bits32(y32))
    for r in sorted({0, 4, R // 2, R - 1}):
        y1 = q4.qmv_rows(p, N, K, x32[r : r + 1])
        torch.cuda.synchronize()
        assert np.array_equal(bits32(y1)[0], bits32(y32)[r]), r
