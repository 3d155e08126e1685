"""Inputs for the op test of the device SwiGLU gate (TensorFold PR #1696,
"What it adds" > Kernels without DPAS: each kernel, SwiGLU among them, gets
an FP64 op test and a planted control).

A 64-wide weight (one group) driven by a one-hot activation x = e_0 gives
every output column n the gate argument a[n] = fl32(s[n] * q[n] + b[n]),
from that column's scale s, code q = code 0 and bias b; a second weight with
scale 0 and bias 1 gives c = 1, so the fused output is silu(a) * 1 = silu(a).
This module only chooses the (s, q, b) triples; the test forms a from them.

The triples cover, for both signs: bf16 magnitudes spread evenly in log scale
from 2^-126 to 2^7; a dense grid over [-100, 100]; the float32 values within
a few thousand ulps of the clamp points -80 and 88 and of -88, 80, -64, 20;
and very large magnitudes (silu(a) = a or -0 there).
"""

from __future__ import annotations

import numpy as np

import synthetic

K = 64


def _bf16(v):
    return synthetic.bf16_bits_from_f64(np.asarray(v, dtype=np.float64))


def bf16_value(bits):
    """The value of bf16 patterns (their bits are the top half of a float32)."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def cases(seed: int = 11, n: int = 16384):
    """Triples (s_bits, q, b_bits) of bf16 patterns and codes 1..15, n of
    them (a multiple of 64)."""
    rng = np.random.default_rng(seed)
    s, q, b = [], [], []
    # 1. bf16 grid, log-uniform magnitudes 2^-126 .. 2^7, random sign
    m = n // 4
    mag = np.exp2(rng.uniform(-126.0, 7.0, m))
    s.append(_bf16(mag * rng.choice([-1.0, 1.0], m)))
    q.append(np.ones(m, dtype=np.uint8))
    b.append(np.zeros(m, dtype=np.uint16))
    # 2. dense grid over [-100, 100]: a bf16 bias plus a small multiple of
    #    twice its float32 ulp, so a is a float32 with more than 8 significant
    #    bits and s * q + b is exact in float32 (every rounding mode agrees)
    m = n // 4
    bv = rng.uniform(-100.0, 100.0, m)
    bb = _bf16(bv)
    b.append(bb)
    ulp = np.exp2(np.floor(np.log2(np.abs(bf16_value(bb)))) - 23.0)
    s.append(_bf16(2.0 * ulp * rng.integers(1, 256, m) * rng.choice([-1.0, 1.0], m)))
    q.append(rng.integers(1, 16, m).astype(np.uint8))
    # 3. ulp neighbourhoods of the clamp points and other landmarks: a float32
    #    ulp in [64, 128) is 2^-17 and in [16, 32) 2^-19
    m = n // 4
    centers = np.array([-80.0, 88.0, -88.0, 80.0, -64.0, 20.0])
    ulp = np.where(np.abs(centers) >= 64.0, 2.0 ** -17, 2.0 ** -19)
    pick = rng.integers(0, len(centers), m)
    b.append(_bf16(centers[pick]))
    s.append(_bf16(ulp[pick] * rng.integers(1, 256, m) * rng.choice([-1.0, 1.0], m)))
    q.append(rng.integers(1, 16, m).astype(np.uint8))
    # 4. the rest: large magnitudes up to 2^120 and the exact landmarks
    m = n - sum(len(v) for v in s)
    big = np.exp2(rng.uniform(7.0, 120.0, m)) * rng.choice([-1.0, 1.0], m)
    big[:12] = [-80.0, 88.0, -88.0, 80.0, 0.5, -0.5, 1.0, -1.0, 2.0 ** -126, -(2.0 ** -126), 100.0, -100.0]
    s.append(_bf16(big))
    q.append(np.ones(m, dtype=np.uint8))
    b.append(np.zeros(m, dtype=np.uint16))
    return np.concatenate(s), np.concatenate(q), np.concatenate(b)


def weights(seed: int = 11, n: int = 16384):
    """(w_a, w_c, x): w_a holds the triples in group 0 with code q at k = 0
    (the other codes random: x is zero there), w_c has scale 0 and bias 1,
    x is one bf16 row e_0."""
    s_bits, q0, b_bits = cases(seed, n)
    rng = np.random.default_rng(seed + 1)
    codes = rng.integers(0, 16, (n, K), dtype=np.uint8)
    codes[:, 0] = q0
    wa = synthetic.QWeight("silu_a", n, K, synthetic.pack_codes_low_nibble_first(codes), s_bits.reshape(n, 1), b_bits.reshape(n, 1))
    one = _bf16(np.ones((n, 1)))
    zero = np.zeros((n, 1), dtype=np.uint16)
    wc = synthetic.QWeight("silu_c", n, K, synthetic.pack_codes_low_nibble_first(codes), zero, one)
    x = np.zeros((1, K), dtype=np.uint16)
    x[0, 0] = _bf16(1.0)
    return wa, wc, x
