"""Pins for the float64 oracle: facts fixed by the pages and by mathematics,
chosen so a plausible mistake in the oracle (wrong nibble order, wrong group
index, dropped bias, swapped scale/bias, transposed operand, wrong silu sign)
fails at least one of them. No GPU needed."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic
from tests.tolerance import tol_loosest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(v):
    return synthetic.bf16_bits_from_f64(np.asarray(v, dtype=np.float64))


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- unpacking


def test_unpack_hand_worked_words():
    for case in _load("unpack_words.json")["cases"]:
        word = np.array([[int(case["word"], 16)]], dtype=np.uint32)
        q = oracle.unpack_codes(word, 8)
        assert q.tolist() == [case["codes"]], case


def test_unpack_multiword_row_order():
    # two rows, two words each: code k of row n is at word k//8, nibble k%8
    wq = np.array([[0x76543210, 0xFEDCBA98], [0x01234567, 0x89ABCDEF]], dtype=np.uint32)
    q = oracle.unpack_codes(wq, 16)
    assert q[0].tolist() == list(range(16))
    assert q[1].tolist() == [7, 6, 5, 4, 3, 2, 1, 0, 15, 14, 13, 12, 11, 10, 9, 8]


# ------------------------------------------------------------ dequantization


def test_dequant_hand_worked():
    for case in _load("dequant_cases.json")["cases"]:
        s = np.full((1, 1), int(case["scale_bits"], 16), dtype=np.uint16)
        b = np.full((1, 1), int(case["bias_bits"], 16), dtype=np.uint16)
        q = np.full((1, 64), case["q"], dtype=np.uint8)
        wq = synthetic.pack_codes_low_nibble_first(q)
        w = oracle.dequantize(wq, s, b, 64)
        assert np.all(w == case["w"]), case


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x8000, 0x3F00, 0x7F7F], dtype=np.uint16)
    v = oracle.bf16_to_f64(bits)
    assert v[:6].tolist() == [1.0, -1.0, 2.0, 0.0, -0.0, 0.5]
    assert math.copysign(1.0, v[4]) == -1.0
    assert v[6] == float.fromhex("0x1.fe00000000000p+127")


# ------------------------------------------------------------- closed forms


def _random_weight(rng, N, K, scale_sign_mix=True):
    q = rng.integers(0, 16, (N, K), dtype=np.uint8)
    s = np.abs(rng.normal(0, 0.02, (N, K // 64)))
    if scale_sign_mix:
        s *= rng.choice([-1.0, 1.0, 0.0], size=s.shape, p=[0.3, 0.6, 0.1])
    sb = _bf16(s)
    bb = _bf16(rng.normal(0, 0.2, (N, K // 64)))
    return q, synthetic.pack_codes_low_nibble_first(q), sb, bb


@pytest.mark.parametrize("k", [0, 1, 7, 8, 31, 32, 63, 64, 65, 127, 128, 255])
def test_one_hot_activation_picks_one_weight(k):
    """x = e_k gives y[n] = s[n][k//64] * q[n][k] + b[n][k//64]; k=32 separates
    64-wide groups from 32-wide ones, k=63/64 sits on a group boundary."""
    rng = np.random.default_rng(100 + k)
    N, K = 16, 256
    q, wq, sb, bb = _random_weight(rng, N, K)
    x = np.zeros((1, K), dtype=np.uint16)
    x[0, k] = 0x3F80  # 1.0
    y = oracle.matmul_rows(wq, sb, bb, x)[0]
    s = oracle.bf16_to_f64(sb)[:, k // 64]
    b = oracle.bf16_to_f64(bb)[:, k // 64]
    assert np.array_equal(y, s * q[:, k].astype(np.float64) + b)


def _group_code_sums_bytewise(wq, K):
    """Sum of codes per (row, group) computed bytewise from the words (an
    independent path from the oracle's shift-per-code unpack)."""
    words = wq.astype(np.uint64)
    lo = words & 0x0F0F0F0F
    hi = (words >> 4) & 0x0F0F0F0F
    per_word = np.zeros(words.shape, dtype=np.int64)
    for byte in range(4):
        per_word += ((lo >> (8 * byte)) & 0xFF).astype(np.int64)
        per_word += ((hi >> (8 * byte)) & 0xFF).astype(np.int64)
    return per_word.reshape(wq.shape[0], K // 64, 8).sum(axis=2)


def test_all_ones_activation_closed_form():
    rng = np.random.default_rng(7)
    N, K = 24, 512
    _, wq, sb, bb = _random_weight(rng, N, K)
    x = np.full((1, K), 0x3F80, dtype=np.uint16)
    y = oracle.matmul_rows(wq, sb, bb, x)[0]
    qsum = _group_code_sums_bytewise(wq, K).astype(np.float64)
    s = oracle.bf16_to_f64(sb)
    b = oracle.bf16_to_f64(bb)
    terms = s * qsum + 64.0 * b  # each exact: s*qsum has <= 8+10 bits
    expect = np.array([math.fsum(r) for r in terms])
    A = oracle.error_weight(wq, sb, bb, x)[0]
    assert np.all(np.abs(y - expect) <= (K + 2) * 2.0 ** -52 * A)


def test_integer_weights_reduce_to_integer_matmul():
    """With s=1, b=0 the weights are the codes; with small-integer x the
    product is an exact integer matrix product (int64 matmul)."""
    rng = np.random.default_rng(11)
    N, K, M = 20, 192, 3
    q, wq, _, _ = _random_weight(rng, N, K)
    sb = np.full((N, K // 64), 0x3F80, dtype=np.uint16)
    bb = np.zeros((N, K // 64), dtype=np.uint16)
    xi = rng.integers(-8, 9, (M, K))
    x = _bf16(xi.astype(np.float64))
    y = oracle.matmul_rows(wq, sb, bb, x)
    assert np.array_equal(y, (xi @ q.astype(np.int64).T).astype(np.float64))


def test_rectangular_shapes_and_orientation():
    """y is [M][N]; row m only depends on x[m] and column n only on weight row n."""
    rng = np.random.default_rng(12)
    N, K, M = 8, 128, 3
    _, wq, sb, bb = _random_weight(rng, N, K)
    x = _bf16(rng.normal(0, 1, (M, K)))
    y = oracle.matmul_rows(wq, sb, bb, x)
    assert y.shape == (M, N)
    y_row1 = oracle.matmul_rows(wq, sb, bb, x[1:2])
    y_col5 = oracle.matmul_rows(wq[5:6], sb[5:6], bb[5:6], x)
    assert np.array_equal(y[1:2], y_row1)
    assert np.array_equal(y[:, 5:6], y_col5)


# ------------------------------------------------------- exact brute force


@pytest.mark.parametrize("seed,N,K,M", [(1, 4, 64, 1), (2, 8, 128, 3), (3, 3, 256, 2)])
def test_fsum_equals_fraction_bruteforce(seed, N, K, M):
    rng = np.random.default_rng(seed)
    _, wq, sb, bb = _random_weight(rng, N, K)
    x = _bf16(rng.normal(0, 1, (M, K)) * rng.choice([1e-3, 1.0, 30.0], (M, K)))
    exact = oracle.matmul_rows_fraction(wq, sb, bb, x)
    fs = oracle.matmul_rows_exact(wq, sb, bb, x)
    for i in range(M):
        for n in range(N):
            assert fs[i, n] == float(exact[i][n])  # fsum is correctly rounded


def test_fraction_bruteforce_float32_activations():
    rng = np.random.default_rng(4)
    N, K, M = 3, 128, 2
    _, wq, sb, bb = _random_weight(rng, N, K)
    x = rng.normal(0, 1, (M, K)).astype(np.float32)
    exact = oracle.matmul_rows_fraction(wq, sb, bb, x)
    fs = oracle.matmul_rows_exact(wq, sb, bb, x)
    for i in range(M):
        for n in range(N):
            assert fs[i, n] == float(exact[i][n])


@pytest.mark.parametrize("cfg", [0, 2])
def test_dgemm_within_float64_bound_of_exact(cfg):
    data = synthetic.config(cfg)
    w = data["w"] if cfg == 0 else data["wq"]
    x = data["x"][:4]
    cols = np.arange(0, w.N, max(1, w.N // 48))
    y = oracle.matmul_rows(w.wq, w.scales, w.biases, x, cols=cols)
    ye = oracle.matmul_rows_exact(w.wq, w.scales, w.biases, x, cols=cols)
    A = oracle.error_weight(w.wq, w.scales, w.biases, x, cols=cols)
    assert np.all(np.abs(y - ye) <= (w.K + 2) * 2.0 ** -52 * A)
    # and the exact sums are genuinely non-trivial
    assert np.all(np.abs(ye) > 0)


def test_error_weight_dominates_and_is_tight_for_positive_data():
    rng = np.random.default_rng(5)
    N, K = 6, 128
    q = rng.integers(0, 16, (N, K), dtype=np.uint8)
    wq = synthetic.pack_codes_low_nibble_first(q)
    sb = _bf16(np.abs(rng.normal(0, 0.1, (N, 2))))
    bb = _bf16(np.abs(rng.normal(0, 0.1, (N, 2))))
    x = _bf16(np.abs(rng.normal(0, 1, (2, K))))
    y = oracle.matmul_rows(wq, sb, bb, x)
    A = oracle.error_weight(wq, sb, bb, x)
    assert np.allclose(y, A, rtol=1e-14, atol=0)  # all terms positive: A == y
    x2 = _bf16(rng.normal(0, 1, (2, K)))
    assert np.all(np.abs(oracle.matmul_rows(wq, sb, bb, x2)) <= oracle.error_weight(wq, sb, bb, x2))


# ------------------------------------------------------------------ SwiGLU


def test_silu_identities():
    a = np.array([0.0, 0.5, -0.5, 3.0, -3.0, 12.5, -12.5])
    s = oracle.silu(a)
    assert s[0] == 0.0
    # silu(-a) = silu(a) - a
    assert np.allclose(oracle.silu(-a), s - a, rtol=0, atol=1e-15)
    # silu(a) -> a for large a, -> -0 for very negative a
    assert oracle.silu(np.array([40.0]))[0] == 40.0
    big_neg = oracle.silu(np.array([-800.0]))[0]
    assert big_neg == 0.0 and math.copysign(1.0, big_neg) == -1.0
    # silu(1) = 1 / (1 + 1/e)
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    # closed form at log(3): sigmoid = 3/4
    assert abs(oracle.silu(np.array([math.log(3.0)]))[0] - 0.75 * math.log(3.0)) < 1e-15


def test_swiglu_is_silu_of_first_times_second():
    a = np.array([1.0, -2.0, 0.0, 4.0])
    c = np.array([2.0, 3.0, 5.0, -0.5])
    z = oracle.swiglu(a, c)
    assert z[2] == 0.0
    assert abs(z[0] - 2.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(z[1] - 3.0 * (-2.0) / (1.0 + math.exp(2.0))) < 1e-15
    # not symmetric: swapping the operands changes the value
    assert not np.allclose(oracle.swiglu(c, a), z)


# ------------------------------------------------------- planted mistakes


def _plant(kind, wq, sb, bb, K):
    """Oracle variants with one planted mistake each (the pages' own control
    is the other group size; the rest are the natural slips)."""
    q = oracle.unpack_codes(wq, K).astype(np.float64)
    s = oracle.bf16_to_f64(sb)
    b = oracle.bf16_to_f64(bb)
    G = K // 64
    g = np.arange(K) // 64
    if kind == "group32":
        g = np.minimum(np.arange(K) // 32, G - 1)
        return s[:, g] * q + b[:, g]
    if kind == "high_nibble_first":
        k = np.arange(K)
        words = np.asarray(wq, dtype=np.uint32)[:, k // 8]
        qh = ((words >> (4 * (7 - k % 8)).astype(np.uint32)) & 0xF).astype(np.float64)
        return s[:, g] * qh + b[:, g]
    if kind == "bias_dropped":
        return s[:, g] * q
    if kind == "scale_bias_swapped":
        return b[:, g] * q + s[:, g]
    if kind == "w_rounded_bf16":
        return oracle.bf16_to_f64(_bf16(s[:, g] * q + b[:, g]))
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["group32", "high_nibble_first", "bias_dropped", "scale_bias_swapped", "w_rounded_bf16"])
@pytest.mark.parametrize("cfg", [0, 2])
def test_planted_mistakes_fail_the_tolerance(kind, cfg):
    data = synthetic.config(cfg)
    w = data["w"] if cfg == 0 else data["wq"]
    x = data["x"][:4]
    cols = np.arange(0, w.N, 4)
    wq, sb, bb = w.wq[cols], w.scales[cols], w.biases[cols]
    y = oracle.matmul_rows(wq, sb, bb, x)
    A = oracle.error_weight(wq, sb, bb, x)
    W_bad = _plant(kind, wq, sb, bb, w.K)
    y_bad = oracle.activations_f64(x) @ W_bad.T
    ratio = np.max(np.abs(y_bad - y) / tol_loosest(A, w.K))
    assert ratio > 1.0, (kind, cfg, ratio)


# ------------------------------------------------- 6- and 8-bit codes (MLX)
# The pages name the 6- and 8-bit checkpoints (PR #1514, "What changes") but
# give no layout; the reading is a little-endian bit stream per row, code k
# at bits bits*k .. bits*k + bits - 1.


def _stream_words(codes, bits):
    """Words of a row built with Python integers: an independent derivation
    of the bit-stream layout (no numpy shifts, no per-word loop)."""
    v = 0
    for k, c in enumerate(codes):
        v |= int(c) << (bits * k)
    nwords = len(codes) * bits // 32
    return np.array([[(v >> (32 * j)) & 0xFFFFFFFF for j in range(nwords)]], dtype=np.uint32)


def test_unpack_6bit_straddling_hand_worked():
    # code 5 of a row: bits 30..35, so 0b111111 is the top two bits of word 0
    # (0xC0000000) and the low four of word 1 (0x0000000F)
    q = oracle.unpack_codes(np.array([[0xC0000000, 0x0000000F, 0]], dtype=np.uint32), 16, 6)
    assert q[0].tolist() == [0] * 5 + [63] + [0] * 10
    # code 10: bits 60..65; 42 = 0b101010 puts 0b1010 at the top of word 1
    # and 0b10 at the bottom of word 2
    q = oracle.unpack_codes(np.array([[0, 0xA0000000, 0x2]], dtype=np.uint32), 16, 6)
    assert q[0].tolist() == [0] * 10 + [42] + [0] * 5
    # all bits set: every code is 63
    q = oracle.unpack_codes(np.full((1, 3), 0xFFFFFFFF, dtype=np.uint32), 16, 6)
    assert q[0].tolist() == [63] * 16


@pytest.mark.parametrize("bits", [6, 8])
def test_unpack_single_code_walk(bits):
    """Each code position alone at its maximum, then a value pattern; the
    words come from Python integer arithmetic."""
    K = 64
    top = (1 << bits) - 1
    for k in range(K):
        codes = [0] * K
        codes[k] = top
        assert oracle.unpack_codes(_stream_words(codes, bits), K, bits)[0].tolist() == codes, k
    codes = [(7 * k + 3) % (1 << bits) for k in range(K)]
    assert oracle.unpack_codes(_stream_words(codes, bits), K, bits)[0].tolist() == codes


def test_unpack_8bit_is_bytes_in_order():
    q = oracle.unpack_codes(np.array([[0x04030201, 0xFFEE8000]], dtype=np.uint32), 8, 8)
    assert q[0].tolist() == [1, 2, 3, 4, 0x00, 0x80, 0xEE, 0xFF]


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_generator_packer_and_oracle_unpack_agree(bits):
    """The generator's chunked packer and the oracle's bit-position unpack are
    written independently; they must invert each other."""
    rng = np.random.default_rng(40 + bits)
    q = rng.integers(0, 1 << bits, (5, 320), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_codes(synthetic.pack_codes_bits(q, bits), 320, bits), q)


def _random_weight_bits(rng, N, K, bits):
    q = rng.integers(0, 1 << bits, (N, K), dtype=np.uint8)
    s = np.abs(rng.normal(0, 0.02, (N, K // 64))) * rng.choice([-1.0, 1.0, 0.0], size=(N, K // 64), p=[0.3, 0.6, 0.1])
    return q, synthetic.pack_codes_bits(q, bits), _bf16(s), _bf16(rng.normal(0, 0.2, (N, K // 64)))


@pytest.mark.parametrize("bits", [6, 8])
@pytest.mark.parametrize("k", [0, 5, 31, 63, 64, 127])
def test_one_hot_activation_picks_one_weight_bits(bits, k):
    rng = np.random.default_rng(200 + 10 * bits + k)
    N, K = 8, 128
    q, wq, sb, bb = _random_weight_bits(rng, N, K, bits)
    x = np.zeros((1, K), dtype=np.uint16)
    x[0, k] = 0x3F80
    y = oracle.matmul_rows(wq, sb, bb, x, bits=bits)[0]
    s = oracle.bf16_to_f64(sb)[:, k // 64]
    b = oracle.bf16_to_f64(bb)[:, k // 64]
    assert np.array_equal(y, s * q[:, k].astype(np.float64) + b)


@pytest.mark.parametrize("bits", [6, 8])
def test_integer_weights_reduce_to_integer_matmul_bits(bits):
    rng = np.random.default_rng(300 + bits)
    N, K, M = 12, 192, 3
    q, wq, _, _ = _random_weight_bits(rng, N, K, bits)
    sb = np.full((N, K // 64), 0x3F80, dtype=np.uint16)
    bb = np.zeros((N, K // 64), dtype=np.uint16)
    xi = rng.integers(-8, 9, (M, K))
    y = oracle.matmul_rows(wq, sb, bb, _bf16(xi.astype(np.float64)), bits=bits)
    assert np.array_equal(y, (xi @ q.astype(np.int64).T).astype(np.float64))


@pytest.mark.parametrize("bits", [6, 8])
def test_fsum_equals_fraction_bruteforce_bits(bits):
    """Exact products summed by fsum against Fraction sums whose codes are read
    one bit at a time from the words."""
    rng = np.random.default_rng(400 + bits)
    N, K, M = 3, 128, 2
    _, wq, sb, bb = _random_weight_bits(rng, N, K, bits)
    x = _bf16(rng.normal(0, 1, (M, K)))
    exact = oracle.matmul_rows_exact(wq, sb, bb, x, bits=bits)
    frac = oracle.matmul_rows_fraction(wq, sb, bb, x, bits=bits)
    for m in range(M):
        for n in range(N):
            assert exact[m, n] == float(frac[m][n])
    y = oracle.matmul_rows(wq, sb, bb, x, bits=bits)
    A = oracle.error_weight(wq, sb, bb, x, bits=bits)
    assert np.all(np.abs(y - exact) <= (K + 2) * 2.0 ** -52 * A)


def test_6bit_read_without_straddling_fails():
    """A plausible mistake, planted in a copy of the decode: 6-bit codes read
    as five per word (never straddling) disagree with the exact sums by far
    more than the fp32 tolerance."""
    rng = np.random.default_rng(500)
    N, K = 4, 64
    q, wq, sb, bb = _random_weight_bits(rng, N, K, 6)
    wrong = np.zeros_like(q)
    for k in range(K):
        word = wq[:, k // 5] if k // 5 < wq.shape[1] else np.zeros(N, dtype=np.uint32)
        wrong[:, k] = (word >> np.uint32(6 * (k % 5))) & 0x3F
    x = _bf16(rng.normal(0, 1, (1, K)))
    exact = oracle.matmul_rows_exact(wq, sb, bb, x, bits=6)
    wrong_wq = synthetic.pack_codes_bits(wrong, 6)
    y_wrong = oracle.matmul_rows(wrong_wq, sb, bb, x, bits=6)
    T = tol_loosest(oracle.error_weight(wq, sb, bb, x, bits=6), K)
    assert np.any(np.abs(y_wrong - exact) > T)


# ------------------------------------------------ block FP8 (weight-only)
# PR #1696 serves "the block FP8 export weight-only"; the reading is OCP E4M3
# bytes with a float32 scale per 128 x 128 block.


def test_e4m3_hand_worked_values():
    table = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
             0x08: 2.0 ** -6, 0x77: 240.0, 0xB8: -1.0, 0xFE: -448.0, 0x30: 0.5}
    codes = np.array(list(table), dtype=np.uint8)
    assert oracle.e4m3_to_f64(codes).tolist() == list(table.values())
    assert math.copysign(1.0, float(oracle.e4m3_to_f64(np.array([0x80], dtype=np.uint8))[0])) == -1.0
    assert np.all(np.isnan(oracle.e4m3_to_f64(np.array([0x7F, 0xFF], dtype=np.uint8))))


def test_e4m3_all_codes_by_accumulated_steps():
    """Positive codes in order differ by 2^-9 below 0x08 and by 2^(e-10)
    within exponent field e: the whole table rebuilt from its increments."""
    expect = [0.0]
    for c in range(1, 0x7F):
        e = c >> 3
        step = 2.0 ** -9 if c <= 8 else 2.0 ** ((c - 1 >> 3) - 10)
        expect.append(expect[-1] + step)
    v = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert v.tolist() == expect
    neg = oracle.e4m3_to_f64(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert (-neg[1:]).tolist() == expect[1:]


def _fp8(rng, N, K):
    return synthetic.draw_fp8_weight(rng, "f", N, K)


@pytest.mark.parametrize("k", [0, 63, 64, 127, 128, 255])
def test_fp8_one_hot_activation_and_block_scales(k):
    rng = np.random.default_rng(600 + k)
    w = _fp8(rng, 256, 256)
    x = np.zeros((1, 256), dtype=np.uint16)
    x[0, k] = 0x3F80
    y = oracle.matmul_rows_fp8(w.w8, w.scales, x)[0]
    vals = oracle.e4m3_to_f64(w.w8[:, k])
    s = w.scales.astype(np.float64)[np.arange(256) // 128, k // 128]
    assert np.array_equal(y, vals * s)
    # rows 127 and 128 sit in different scale blocks
    assert w.scales[0, k // 128] != w.scales[1, k // 128]


def test_fp8_fsum_equals_fraction_bruteforce():
    rng = np.random.default_rng(610)
    w = _fp8(rng, 64, 192)
    w8 = w.w8[:3]
    x = _bf16(rng.normal(0, 1, (2, 192)))
    exact = oracle.matmul_rows_fp8_exact(w8, w.scales[:1], x)
    frac = oracle.matmul_rows_fp8_fraction(w8, w.scales[:1], x)
    for m in range(2):
        for n in range(3):
            assert exact[m, n] == float(frac[m][n])
    y = oracle.matmul_rows_fp8(w8, w.scales[:1], x)
    A = oracle.error_weight_fp8(w8, w.scales[:1], x)
    assert np.all(np.abs(y - exact) <= (192 + 2) * 2.0 ** -52 * A)


def _fp8_error_weight_pins(fn):
    """Facts about A = sum_k |w[n][k]| |x[m][k]| for block-FP8 weights that
    hold by definition; returns the names of those ``fn`` violates.

    * one-hot: x = c * e_k gives A[n] = |e4m3(w8[n][k])| * |s(n, k)| * |c|,
      with scales of both signs and a negative c;
    * all terms positive (positive codes, scales and x): A equals y;
    * A depends on x through |x| only, and A >= |y| for mixed signs."""
    failed = set()
    rng = np.random.default_rng(630)
    N, K = 256, 256
    w = _fp8(rng, N, K)
    sc = w.scales.astype(np.float32).copy()
    sc[1, 0] = -sc[1, 0]  # a negative block scale
    s64 = sc.astype(np.float64)
    for k in (0, 127, 128, 255):
        for c, pat in ((1.5, 0x3FC0), (-2.0, 0xC000)):
            x = np.zeros((1, K), dtype=np.uint16)
            x[0, k] = pat
            A = fn(w.w8, sc, x)[0]
            expect = np.abs(oracle.e4m3_to_f64(w.w8[:, k])) * np.abs(s64[np.arange(N) // 128, k // 128]) * abs(c)
            if not np.array_equal(A, expect):
                failed.add("one_hot")
    wp = (w.w8 & 0x7F).astype(np.uint8)
    wp[wp == 0x7F] = 0x7E
    xp = _bf16(np.abs(rng.normal(0, 1, (2, K))) + 0.01)
    sp = np.abs(w.scales).astype(np.float32)
    yp = oracle.matmul_rows_fp8(wp, sp, xp)
    if not np.allclose(fn(wp, sp, xp), yp, rtol=1e-13, atol=0):
        failed.add("positive_equals_y")
    xm = _bf16(rng.normal(0, 1, (2, K)))
    neg = (xm ^ 0x8000).astype(np.uint16)
    absx = (xm & 0x7FFF).astype(np.uint16)
    A = fn(w.w8, sc, xm)
    if not (np.array_equal(A, fn(w.w8, sc, neg)) and np.array_equal(A, fn(w.w8, sc, absx))):
        failed.add("abs_x")
    if not np.all(np.abs(oracle.matmul_rows_fp8(w.w8, sc, xm)) <= A):
        failed.add("dominates")
    return failed


def test_fp8_error_weight_pins():
    assert _fp8_error_weight_pins(oracle.error_weight_fp8) == set()


def _ew_fp8_planted(kind):
    """error_weight_fp8 with one planted slip."""

    def fn(w8, scales, x):
        X = oracle.activations_f64(x)
        K = X.shape[1]
        w8 = np.asarray(w8, dtype=np.uint8)
        N = w8.shape[0]
        vals = oracle.e4m3_to_f64(w8)
        s = np.asarray(scales, dtype=np.float32).astype(np.float64)[np.arange(N) // 128][:, np.arange(K) // 128]
        if kind == "scale_dropped":
            W = np.abs(vals)
        elif kind == "scale_not_abs":
            W = np.abs(vals) * s
        elif kind == "x_not_abs":
            return X @ (np.abs(vals * s)).T
        elif kind == "w_not_abs":
            W = vals * s
        else:
            raise ValueError(kind)
        return np.abs(X) @ W.T

    return fn


@pytest.mark.parametrize("kind", ["scale_dropped", "scale_not_abs", "x_not_abs", "w_not_abs"])
def test_fp8_error_weight_planted_slips_fail_its_pins(kind):
    assert _fp8_error_weight_pins(_ew_fp8_planted(kind)), kind


@pytest.mark.parametrize("kind", ["bias8", "block64", "e5m2"])
def test_fp8_planted_mistakes_fail(kind):
    """Plausible misreadings of the format, planted in a copy of the decode,
    land far outside the fp32 tolerance."""
    rng = np.random.default_rng(620)
    w = _fp8(rng, 256, 256)
    x = _bf16(rng.normal(0, 1, (2, 256)))
    exact = oracle.matmul_rows_fp8_exact(w.w8, w.scales, x)
    c = w.w8.astype(np.int64)
    if kind == "bias8":
        W = oracle.e4m3_to_f64(w.w8) / 2.0 * w.scales.astype(np.float64)[np.arange(256) // 128][:, np.arange(256) // 128]
    elif kind == "block64":
        W = oracle.e4m3_to_f64(w.w8) * w.scales.astype(np.float64)[np.arange(256) // 64 % 2][:, np.arange(256) // 64 % 2]
    else:
        sign = np.where(c & 0x80, -1.0, 1.0)
        e, m = (c >> 2) & 0x1F, (c & 3).astype(np.float64)
        vals = sign * np.where(e == 0, m / 4 * 2.0 ** -14, (1 + m / 4) * np.exp2(e - 15.0))
        W = vals * w.scales.astype(np.float64)[np.arange(256) // 128][:, np.arange(256) // 128]
    y = oracle.activations_f64(x) @ W.T
    T = tol_loosest(oracle.error_weight_fp8(w.w8, w.scales, x), 256, fmt="fp8")
    assert np.any(np.abs(y - exact) > T)


# --------------------------------------- QK norm, partial RoPE, KV store
# PR #1696 lists QK norm with partial RoPE and a KV ring, and fuses RoPE
# with the KV store on decode; the formulas are readings (half-split pairs,
# angle pos * theta^(-2i/rot)), pinned by the properties that define a
# rotary embedding.


def test_rope_position_zero_and_rot_zero_are_identity():
    rng = np.random.default_rng(800)
    x = rng.normal(0, 1, (3, 4, 64))
    assert np.array_equal(oracle.rope(x, [0, 0, 0], 64, 10000.0), x)
    assert np.array_equal(oracle.rope(x, [5, 9, 100], 0, 10000.0), x)


def test_rope_hand_worked_pair():
    # rot = 2: one pair (0, 1) at angle pos * theta^0 = pos radians
    x = np.zeros((1, 1, 64))
    x[0, 0, 0], x[0, 0, 1], x[0, 0, 5] = 3.0, 4.0, 7.0
    y = oracle.rope(x, [1], 2, 10000.0)[0, 0]
    assert np.allclose(y[0], 3 * math.cos(1) - 4 * math.sin(1), rtol=0, atol=1e-15)
    assert np.allclose(y[1], 4 * math.cos(1) + 3 * math.sin(1), rtol=0, atol=1e-15)
    assert y[5] == 7.0 and np.count_nonzero(y) == 3
    # rot = 4, theta = 16: pairs (0, 2) at pos and (1, 3) at pos / 4
    x = np.zeros((1, 1, 64))
    x[0, 0, 1] = 1.0
    y = oracle.rope(x, [2], 4, 16.0)[0, 0]
    assert np.allclose(y[[1, 3]], [math.cos(0.5), math.sin(0.5)], rtol=0, atol=1e-15)


def test_rope_keeps_pair_norms_and_relative_positions():
    """A rotation keeps every pair's length, and <rope(q, p1), rope(k, p2)>
    depends on p1 - p2 only (the property attention relies on)."""
    rng = np.random.default_rng(801)
    q, k = rng.normal(0, 1, (1, 1, 64)), rng.normal(0, 1, (1, 1, 64))
    rot, h = 48, 24
    qr = oracle.rope(q, [37], rot, 10000.0)
    n0 = q[0, 0, :h] ** 2 + q[0, 0, h:rot] ** 2
    n1 = qr[0, 0, :h] ** 2 + qr[0, 0, h:rot] ** 2
    assert np.allclose(n0, n1, rtol=1e-14, atol=0)
    assert np.array_equal(qr[0, 0, rot:], q[0, 0, rot:])
    dots = [float(np.sum(oracle.rope(q, [p + 11], rot, 10000.0) * oracle.rope(k, [p], rot, 10000.0))) for p in (0, 5, 1000, 65536)]
    assert np.allclose(dots, dots[0], rtol=1e-12, atol=1e-12)


def test_rms_norm_closed_forms():
    x = np.full((1, 64), 3.0)
    assert np.allclose(oracle.rms_norm(x, np.ones(64), 0.0), 1.0, rtol=1e-15)
    g = np.arange(64, dtype=np.float64)
    assert np.allclose(oracle.rms_norm(-x, g, 0.0), -g, rtol=1e-15)
    rng = np.random.default_rng(802)
    y = oracle.rms_norm(rng.normal(0, 5, (7, 64)), np.ones(64), 1e-6)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-6)


def test_rope_kv_splits_heads_in_order():
    rng = np.random.default_rng(803)
    n_q, n_kv = 4, 2
    qkv = rng.normal(0, 1, (2, (n_q + 2 * n_kv) * 64))
    q, k, v = oracle.rope_kv(qkv, [0, 0], n_q, n_kv, 64, 10000.0)
    assert np.array_equal(q, qkv[:, :256])
    assert np.array_equal(k.reshape(2, -1), qkv[:, 256:384])
    assert np.array_equal(v.reshape(2, -1), qkv[:, 384:512])


def test_attention_gate_is_the_section_after_v():
    """Gated attention's fourth matvec (PR #1696, "What it adds": gated GQA): the gate heads follow the v heads in
    the stacked output and pass through the epilogue unchanged; appending them changes nothing for q, k and v."""
    rng = np.random.default_rng(804)
    n_q, n_kv, n_gate = 4, 2, 3
    qkvg = rng.normal(0, 1, (3, (n_q + 2 * n_kv + n_gate) * 64))
    gate = oracle.attention_gate(qkvg, n_q, n_kv, n_gate)
    assert gate.shape == (3, n_gate * 64)
    assert np.array_equal(gate, qkvg[:, 512:704])
    pos = [3, 70, 1000]
    with_gate = oracle.rope_kv(qkvg, pos, n_q, n_kv, 48, 10000.0, np.ones(64), np.ones(64))
    without = oracle.rope_kv(qkvg[:, :512], pos, n_q, n_kv, 48, 10000.0, np.ones(64), np.ones(64))
    for a, b in zip(with_gate, without):
        assert np.array_equal(a, b)
    assert oracle.attention_gate(qkvg, n_q, n_kv, 0).shape == (3, 0)
