"""Seeded, synthetic, LFM3-1.7B-shaped inputs in the canonical MLX q4g64 format.

Canonical weight format (the MLX affine 4-bit, group-64 checkpoint layout that
the Intel and Metal LFM3 backends read "as stored"; PR #1696 "What it adds",
PR #1514 "What changes"):

* ``wq``     uint32 ``[N][K/8]``: code k of output row n sits in bits
  ``4*(k%8) .. 4*(k%8)+3`` of word ``k//8`` (low nibble first);
* ``scales`` uint16 ``[N][K/64]``: bf16 bit patterns, one per 64-wide group;
* ``biases`` uint16 ``[N][K/64]``: bf16 bit patterns, one per 64-wide group.

Activations are bf16 bit patterns (uint16) ``[rows][K]`` or float32 ``[rows][K]``.

Recipe (one ``numpy.random.default_rng(seed)`` per workload, draws in the
order the workload names its tensors, weights first, then activations):

* codes  ``q = rng.integers(0, 16, (N, K), dtype=uint8)``;
* scales ``S = bf16(|rng.normal(0, 0.02, (N, K/64))|)``;
* biases ``B = bf16(-8 * S + rng.normal(0, 0.002, (N, K/64)))`` (uses the
  already rounded scale, so codes are centred near 8);
* activations ``X = bf16(rng.normal(0, 1, (rows, K)))``.

Wider codes (bits = 6 or 8; PR #1514, "What changes", serves the MLX 4-, 6-
and 8-bit checkpoints as stored; the pages give no layout or statistics):

* ``wq`` uint32 ``[N][K*bits/32]``: the words of a row are one little-endian
  bit stream and code k occupies bits ``bits*k .. bits*k+bits-1`` (8-bit codes
  are the bytes of each word in order; 6-bit codes straddle words);
* codes ``q = rng.integers(0, 2**bits, (N, K))``;
* scales ``S = bf16(|rng.normal(0, 0.02)| * 15 / (2**bits - 1))`` so that the
  weight range matches the 4-bit recipe;
* biases ``B = bf16(-2**(bits-1) * S + rng.normal(0, 0.002))``.

For bits = 4 these are exactly the draws above.

``bf16(v)`` rounds float64 -> float32 (round to nearest even) -> bf16 (round
to nearest even on the bit pattern). Nothing here unpacks, dequantizes or
multiplies: those steps belong to the oracle and to the kernels.
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

GROUP = 64

CONFIG_NAMES = {
    0: "single q4g64 matvec N=512 K=256 R=1",
    1: "decode FFN: w1/w3 8192x2048 + SwiGLU, then w2 2048x8192, R=1",
    2: "decode attention projections: qkv 3072x2048 + o 2048x2048, R=1..16",
    3: "prefill window GEMM: 1000 rows through w1/w3 8192x2048 + SwiGLU",
    4: "long-prompt layer: 8192 rows through qkv/o/w1/w3/w2 + 65536x2048 head",
}


def bf16_bits_from_f64(v: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bf16 bit pattern (RNE), as uint16."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def pack_codes_low_nibble_first(q: np.ndarray) -> np.ndarray:
    """Store codes [N][K] (values 0..15) as uint32 [N][K/8], code k at bits 4*(k%8)."""
    q = np.asarray(q, dtype=np.uint32)
    n, k = q.shape
    if k % 8:
        raise ValueError("K must be a multiple of 8")
    q = q.reshape(n, k // 8, 8)
    words = np.zeros((n, k // 8), dtype=np.uint32)
    for j in range(8):
        words |= q[:, :, j] << np.uint32(4 * j)
    return words


def pack_codes_bits(q: np.ndarray, bits: int) -> np.ndarray:
    """Store codes [N][K] (values < 2**bits) as uint32 [N][K*bits/32], code k
    at bits bits*k .. of the row's little-endian bit stream."""
    if bits == 4:
        return pack_codes_low_nibble_first(q)
    q = np.asarray(q, dtype=np.uint64)
    n, k = q.shape
    per = 32 // np.gcd(bits, 32)  # codes per whole number of words
    wper = per * bits // 32
    if k % per:
        raise ValueError(f"K must be a multiple of {per} for {bits}-bit codes")
    q = q.reshape(n, k // per, per)
    words = np.zeros((n, k // per, wper), dtype=np.uint64)
    for j in range(per):
        p = bits * j
        w, sh = p // 32, p % 32
        words[:, :, w] |= (q[:, :, j] << np.uint64(sh)) & np.uint64(0xFFFFFFFF)
        if sh + bits > 32:
            words[:, :, w + 1] |= q[:, :, j] >> np.uint64(32 - sh)
    return words.reshape(n, k // per * wper).astype(np.uint32)


@dataclass
class QWeight:
    """One q4g64 matrix in the canonical format."""

    name: str
    N: int
    K: int
    wq: np.ndarray  # uint32 [N][K/8]
    scales: np.ndarray  # uint16 bf16 bits [N][K/64]
    biases: np.ndarray  # uint16 bf16 bits [N][K/64]
    bits: int = 4


def draw_qweight(rng: np.random.Generator, name: str, N: int, K: int, bits: int = 4) -> QWeight:
    if K % GROUP or N <= 0 or K <= 0:
        raise ValueError("K must be a positive multiple of 64 and N positive")
    if bits not in (4, 6, 8):
        raise ValueError("bits must be 4, 6 or 8")
    q = rng.integers(0, 1 << bits, (N, K), dtype=np.uint8)
    if bits == 4:
        s_bits = bf16_bits_from_f64(np.abs(rng.normal(0.0, 0.02, (N, K // GROUP))))
    else:
        s_bits = bf16_bits_from_f64(np.abs(rng.normal(0.0, 0.02, (N, K // GROUP))) * (15.0 / ((1 << bits) - 1)))
    s_val = (s_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    b_bits = bf16_bits_from_f64(-float(1 << (bits - 1)) * s_val + rng.normal(0.0, 0.002, (N, K // GROUP)))
    return QWeight(name, N, K, pack_codes_bits(q, bits), s_bits, b_bits, bits)


@dataclass
class FP8Weight:
    """One block-FP8 matrix: OCP E4M3 bytes and a float32 scale per 128 x 128 block."""

    name: str
    N: int
    K: int
    w8: np.ndarray  # uint8 [N][K]
    scales: np.ndarray  # float32 [ceil(N/128)][ceil(K/128)]


def draw_fp8_weight(rng: np.random.Generator, name: str, N: int, K: int) -> FP8Weight:
    """Block-FP8 weights drawn in the code domain (no quantizer): a random
    sign, an exponent field round(normal(7, 2)) clipped to 0..15 and a
    uniform mantissa, the NaN pattern replaced by the largest finite value;
    block scales float32(0.02 * 2**normal(0, 0.5))."""
    if K % GROUP or N % GROUP or N <= 0 or K <= 0:
        raise ValueError("N and K must be positive multiples of 64")
    sign = rng.integers(0, 2, (N, K), dtype=np.uint8)
    e = np.clip(np.rint(rng.normal(7.0, 2.0, (N, K))), 0, 15).astype(np.uint8)
    m = rng.integers(0, 8, (N, K), dtype=np.uint8)
    m = np.where((e == 15) & (m == 7), 6, m).astype(np.uint8)
    w8 = ((sign << 7) | (e << 3) | m).astype(np.uint8)
    sc = (0.02 * np.exp2(rng.normal(0.0, 0.5, (-(-N // 128), -(-K // 128))))).astype(np.float32)
    return FP8Weight(name, N, K, w8, sc)


def draw_bf16_rows(rng: np.random.Generator, rows: int, K: int, sigma: float = 1.0) -> np.ndarray:
    return bf16_bits_from_f64(rng.normal(0.0, sigma, (rows, K)))


def draw_f32_rows(rng: np.random.Generator, rows: int, K: int, sigma: float = 1.0) -> np.ndarray:
    """float32 rows with full 24-bit significands (used for the fp32-activation matvec)."""
    return rng.normal(0.0, sigma, (rows, K)).astype(np.float32)


def sha256_of(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def config(i: int, rows: int | None = None) -> dict:
    """Return the tensors of workload ``i`` (0..4) as a dict.

    ``rows`` only shrinks the activation row count of workloads 3 and 4 for
    quick tests; weights are always drawn at full size so the draw order and
    values of every weight are those of the full workload.
    """
    rng = np.random.default_rng(i)
    out: dict = {"seed": i, "name": CONFIG_NAMES[i]}
    if i == 0:
        out["w"] = draw_qweight(rng, "w", 512, 256)
        out["x"] = draw_bf16_rows(rng, 1, 256)
    elif i == 1:
        out["w1"] = draw_qweight(rng, "w1", 8192, 2048)
        out["w3"] = draw_qweight(rng, "w3", 8192, 2048)
        out["w2"] = draw_qweight(rng, "w2", 2048, 8192)
        out["x"] = draw_bf16_rows(rng, 1, 2048)
        # A standalone float32 input for w2 with the scale of a SwiGLU output,
        # drawn after the workload's own tensors so they are unaffected.
        out["x_w2_f32"] = draw_f32_rows(rng, 4, 8192, sigma=0.05)
    elif i == 2:
        out["wq"] = draw_qweight(rng, "wq", 2048, 2048)
        out["wk"] = draw_qweight(rng, "wk", 512, 2048)
        out["wv"] = draw_qweight(rng, "wv", 512, 2048)
        out["wo"] = draw_qweight(rng, "wo", 2048, 2048)
        out["x"] = draw_bf16_rows(rng, 16, 2048)
    elif i == 3:
        out["w1"] = draw_qweight(rng, "w1", 8192, 2048)
        out["w3"] = draw_qweight(rng, "w3", 8192, 2048)
        out["x"] = draw_bf16_rows(rng, 1000 if rows is None else rows, 2048)
        out["cuts"] = {
            "w64": [64] * 15 + [40],
            "w128": [128] * 7 + [104],
            "w256": [256] * 3 + [232],
            "ragged": [17, 300, 683],
        }
    elif i == 4:
        out["wq"] = draw_qweight(rng, "wq", 2048, 2048)
        out["wk"] = draw_qweight(rng, "wk", 512, 2048)
        out["wv"] = draw_qweight(rng, "wv", 512, 2048)
        out["wo"] = draw_qweight(rng, "wo", 2048, 2048)
        out["w1"] = draw_qweight(rng, "w1", 8192, 2048)
        out["w3"] = draw_qweight(rng, "w3", 8192, 2048)
        out["w2"] = draw_qweight(rng, "w2", 2048, 8192)
        out["head"] = draw_qweight(rng, "head", 65536, 2048)
        out["x"] = draw_bf16_rows(rng, 8192 if rows is None else rows, 2048)
        # bf16 stand-in for the SwiGLU output that w2 consumes, for per-op parity.
        out["x_w2_bf16"] = draw_bf16_rows(rng, 256, 8192, sigma=0.05)
    else:
        raise ValueError("workloads are numbered 0..4")
    return out


def concat_rows(*ws: QWeight, name: str = "cat") -> QWeight:
    """Stack several matrices along N (output rows); pure data movement."""
    K = ws[0].K
    if any(w.K != K for w in ws):
        raise ValueError("all matrices must share K")
    if any(w.bits != ws[0].bits for w in ws):
        raise ValueError("all matrices must share bits")
    return QWeight(
        name,
        sum(w.N for w in ws),
        K,
        np.concatenate([w.wq for w in ws]),
        np.concatenate([w.scales for w in ws]),
        np.concatenate([w.biases for w in ws]),
        ws[0].bits,
    )
