"""The attention-side decode epilogue (PR #1696: QK norm with partial RoPE,
a KV ring, and decode fusing RoPE with the KV store) on the GPU.

* The fused call (qmv_qkv_rope) equals qmv_rows followed by rope_kv_store
  bit for bit, and every row equals its one-row call.
* The stand-alone epilogue sits within a derived bound of the float64
  epilogue applied to the same float32 q/k/v values; v is copied exactly;
  the bf16 cache holds the round-to-nearest-even of the float32 cache.
* Only the rows' ring slots are written.
* End to end, q/k/v against the float64 matvec and epilogue.
* Gated attention's fourth matvec: gate heads stacked after v pass through
  both calls unchanged (bit-equal to qmv_rows' columns), leave q/k/v as
  they are without them, and every row equals its one-row call."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import oracle
import synthetic
from tests.gpu_helpers import DEV, bits16, bits32, dev_bf16, dev_weight, host_f64, say
from tests.tolerance import tol

pytestmark = pytest.mark.gpu

NQ, NKV, RING = 32, 8, 64
NG = 32  # gate heads (one per q head)
CASES = [dict(rot=64, theta=1e6, norm=False), dict(rot=32, theta=10000.0, norm=True), dict(rot=0, theta=10000.0, norm=True)]


@pytest.fixture(scope="module")
def c2():
    d = synthetic.config(2)
    d["qkv"] = synthetic.concat_rows(d["wq"], d["wk"], d["wv"], name="qkv")
    d["p"] = dev_weight(d["qkv"])
    d["xd"] = dev_bf16(d["x"])
    rng = np.random.default_rng(950)
    # 16 positions with distinct ring slots, some past the ring length
    d["pos"] = (rng.permutation(RING)[:16] + RING * rng.integers(0, 600, 16)).astype(np.int32)
    d["gq"] = (1.0 + 0.1 * rng.normal(0, 1, 64)).astype(np.float32)
    d["gk"] = (1.0 + 0.1 * rng.normal(0, 1, 64)).astype(np.float32)
    return d


def _outs(R, dtype=torch.float32):
    q = torch.full((R, NQ * 64), float("nan"), device=DEV)
    k = torch.full((RING, NKV, 64), float("nan"), device=DEV, dtype=dtype)
    v = torch.full((RING, NKV, 64), float("nan"), device=DEV, dtype=dtype)
    return q, k, v


def _gammas(c2, case):
    if not case["norm"]:
        return None, None
    return torch.from_numpy(c2["gq"]).to(DEV), torch.from_numpy(c2["gk"]).to(DEV)


def _run(c2, case, R, fused, dtype=torch.float32):
    pos = torch.from_numpy(c2["pos"][:R]).to(DEV)
    gq, gk = _gammas(c2, case)
    q, k, v = _outs(R, dtype)
    w = c2["qkv"]
    if fused:
        q4.qmv_qkv_rope(c2["p"], w.K, c2["xd"][:R], pos, NQ, NKV, case["rot"], case["theta"], q, k, v, gq, gk)
    else:
        y = q4.qmv_rows(c2["p"], w.N, w.K, c2["xd"][:R])
        q4.rope_kv_store(y, pos, NQ, NKV, case["rot"], case["theta"], q, k, v, gq, gk)
    torch.cuda.synchronize()
    return q, k, v


@pytest.mark.parametrize("ci", range(len(CASES)))
@pytest.mark.parametrize("R", [1, 3, 16])
def test_fused_equals_composition(c2, ci, R):
    case = CASES[ci]
    say(f"qmv_qkv_rope R={R} {case}")
    a = _run(c2, case, R, fused=True)
    b = _run(c2, case, R, fused=False)
    for t1, t2 in zip(a, b):
        assert np.array_equal(bits32(t1), bits32(t2))
    # only the rows' slots were written
    slots = set(int(p) % RING for p in c2["pos"][:R])
    written = [s for s in range(RING) if not torch.isnan(a[1][s]).all()]
    assert set(written) == slots


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_fused_rows_equal_one_row(c2, ci):
    case = CASES[ci]
    q16, k16, v16 = _run(c2, case, 16, fused=True)
    for r in (0, 7, 15):
        pos = torch.from_numpy(c2["pos"][r : r + 1]).to(DEV)
        gq, gk = _gammas(c2, case)
        q, k, v = _outs(1)
        w = c2["qkv"]
        q4.qmv_qkv_rope(c2["p"], w.K, c2["xd"][r : r + 1], pos, NQ, NKV, case["rot"], case["theta"], q, k, v, gq, gk)
        torch.cuda.synchronize()
        s = int(c2["pos"][r]) % RING
        assert np.array_equal(bits32(q)[0], bits32(q16)[r])
        assert np.array_equal(bits32(k[s]), bits32(k16[s])) and np.array_equal(bits32(v[s]), bits32(v16[s]))


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_epilogue_within_bound_of_float64(c2, ci):
    """The epilogue's own arithmetic: GPU rope_kv_store on float32 q/k/v
    against the float64 epilogue on the same values. Bound per output:
    16 * 2^-24 * (|x_d| + |x_partner|) of the float64 (normed) inputs, which
    covers the norm (a 64-term butterfly sum, sqrt, reciprocal and two
    products: under 7 units) and the rotation (cos and sin rounded once, a
    product and an fma: under 4 units, on inputs off by under 7 units)."""
    case = CASES[ci]
    R = 16
    w = c2["qkv"]
    y = q4.qmv_rows(c2["p"], w.N, w.K, c2["xd"][:R])
    torch.cuda.synchronize()
    y64 = host_f64(y)
    gq, gk = _gammas(c2, case)
    q, k, v = _outs(R)
    pos = c2["pos"][:R]
    q4.rope_kv_store(y, torch.from_numpy(pos).to(DEV), NQ, NKV, case["rot"], case["theta"], q, k, v, gq, gk)
    torch.cuda.synchronize()
    g64q = None if gq is None else c2["gq"].astype(np.float64)
    g64k = None if gk is None else c2["gk"].astype(np.float64)
    q64, k64, v64 = oracle.rope_kv(y64, pos, NQ, NKV, case["rot"], case["theta"], g64q, g64k, 1e-6)
    # magnitudes of the rotation's inputs (normed values) for the bound
    qin = y64[:, : NQ * 64].reshape(R, NQ, 64)
    kin = y64[:, NQ * 64 : (NQ + NKV) * 64].reshape(R, NKV, 64)
    if case["norm"]:
        qin, kin = oracle.rms_norm(qin, g64q, 1e-6), oracle.rms_norm(kin, g64k, 1e-6)

    def bound(xin):
        a = np.abs(xin)
        rot, h = case["rot"], case["rot"] // 2
        partner = a.copy()
        if rot:
            partner[..., :h], partner[..., h:rot] = a[..., h:rot], a[..., :h]
        else:
            partner[...] = 0.0
        return 16 * 2.0 ** -24 * (a + partner) + 2.0 ** -100

    assert np.all(np.abs(host_f64(q).reshape(R, NQ, 64) - q64.reshape(R, NQ, 64)) <= bound(qin))
    slots = pos % RING
    assert np.all(np.abs(host_f64(k[torch.from_numpy(slots.astype(np.int64))]) - k64) <= bound(kin))
    assert np.array_equal(host_f64(v[torch.from_numpy(slots.astype(np.int64))]), v64)  # v is copied


def test_bf16_cache_is_rne_of_float32(c2):
    case = CASES[1]
    _, k32, v32 = _run(c2, case, 16, fused=True)
    _, kb, vb = _run(c2, case, 16, fused=True, dtype=torch.bfloat16)
    for a, b in ((k32, kb), (v32, vb)):
        slots = [s for s in range(RING) if not torch.isnan(a[s]).all()]
        rne = synthetic.bf16_bits_from_f64(host_f64(a[slots]))
        assert np.array_equal(bits16(b[slots]).view(np.uint16), rne)


def test_end_to_end_against_float64_matvec(c2):
    """No norm: each rotated output is |c| x_d + |s| x_p of matvec outputs,
    so the matvec bound T carries through as |c| T_d + |s| T_p."""
    case = CASES[0]
    R = 4
    w = c2["qkv"]
    q, k, v = _run(c2, case, R, fused=True)
    xs = c2["x"][:R]
    y64 = oracle.matmul_rows(w.wq, w.scales, w.biases, xs)
    T = tol(oracle.error_weight(w.wq, w.scales, w.biases, xs), w.K, order="decode")
    pos = c2["pos"][:R]
    q64, k64, v64 = oracle.rope_kv(y64, pos, NQ, NKV, case["rot"], case["theta"])
    Tq = T[:, : NQ * 64].reshape(R, NQ, 64)
    Tk = T[:, NQ * 64 : (NQ + NKV) * 64].reshape(R, NKV, 64)
    Tv = T[:, (NQ + NKV) * 64 :].reshape(R, NKV, 64)
    yq = y64[:, : NQ * 64].reshape(R, NQ, 64)
    yk = y64[:, NQ * 64 : (NQ + NKV) * 64].reshape(R, NKV, 64)

    def carried(Tx, xin):
        # rot = 64: partner of d is d +- 32; |c|, |s| <= 1
        Tp = np.concatenate([Tx[..., 32:], Tx[..., :32]], axis=-1)
        a = np.abs(xin)
        ap = np.concatenate([a[..., 32:], a[..., :32]], axis=-1)
        return Tx + Tp + 16 * 2.0 ** -24 * (a + ap)

    slots = torch.from_numpy((pos % RING).astype(np.int64))
    assert np.all(np.abs(host_f64(q).reshape(R, NQ, 64) - q64.reshape(R, NQ, 64)) <= carried(Tq, yq))
    assert np.all(np.abs(host_f64(k[slots]) - k64) <= carried(Tk, yk))
    assert np.all(np.abs(host_f64(v[slots]) - v64) <= Tv)


@pytest.fixture(scope="module")
def c2g(c2):
    """config 2's q/k/v with a gate projection of the q projection's shape stacked after v."""
    d = dict(c2)
    wg = synthetic.draw_qweight(np.random.default_rng(951), "wg", NG * 64, 2048)
    d["wg"] = wg
    d["qkvg"] = synthetic.concat_rows(c2["wq"], c2["wk"], c2["wv"], wg, name="qkvg")
    d["pg"] = dev_weight(d["qkvg"])
    return d


def _run_gate(d, case, R, fused, rows=None):
    rows = slice(0, R) if rows is None else rows
    pos = torch.from_numpy(d["pos"][rows]).to(DEV)
    gq, gk = _gammas(d, case)
    q, k, v = _outs(R)
    g = torch.full((R, NG * 64), float("nan"), device=DEV)
    w = d["qkvg"]
    if fused:
        q4.qmv_qkv_rope(d["pg"], w.K, d["xd"][rows], pos, NQ, NKV, case["rot"], case["theta"], q, k, v, gq, gk, gate_out=g)
    else:
        y = q4.qmv_rows(d["pg"], w.N, w.K, d["xd"][rows])
        q4.rope_kv_store(y, pos, NQ, NKV, case["rot"], case["theta"], q, k, v, gq, gk, gate_out=g)
    torch.cuda.synchronize()
    return q, k, v, g


@pytest.mark.parametrize("ci", [0, 1])
@pytest.mark.parametrize("R", [1, 5, 16])
def test_gate_fused_equals_composition(c2g, ci, R):
    case = CASES[ci]
    say(f"qmv_qkv_rope with gate R={R} {case}")
    a = _run_gate(c2g, case, R, fused=True)
    b = _run_gate(c2g, case, R, fused=False)
    for t1, t2 in zip(a, b):
        assert np.array_equal(bits32(t1), bits32(t2))
    # the gate is qmv_rows' gate columns, unchanged; q/k/v are those of the call without a gate
    w = c2g["qkvg"]
    y = q4.qmv_rows(c2g["pg"], w.N, w.K, c2g["xd"][:R])
    torch.cuda.synchronize()
    assert np.array_equal(bits32(a[3]), bits32(y[:, (NQ + 2 * NKV) * 64 :]))
    plain = _run(c2g, case, R, fused=True)
    for t1, t2 in zip(a[:3], plain):
        assert np.array_equal(bits32(t1), bits32(t2))


def test_gate_rows_equal_one_row(c2g):
    case = CASES[1]
    q16, k16, v16, g16 = _run_gate(c2g, case, 16, fused=True)
    for r in (0, 9, 15):
        q, k, v, g = _run_gate(c2g, case, 1, fused=True, rows=slice(r, r + 1))
        s = int(c2g["pos"][r]) % RING
        assert np.array_equal(bits32(g)[0], bits32(g16)[r]) and np.array_equal(bits32(q)[0], bits32(q16)[r])
        assert np.array_equal(bits32(k[s]), bits32(k16[s])) and np.array_equal(bits32(v[s]), bits32(v16[s]))


def test_gate_against_float64_matvec(c2g):
    """The gate is a plain matvec output: within the matvec bound T of the float64 oracle."""
    R = 4
    _, _, _, g = _run_gate(c2g, CASES[0], R, fused=True)
    wg, xs = c2g["wg"], c2g["x"][:R]
    y64 = oracle.matmul_rows(wg.wq, wg.scales, wg.biases, xs)
    T = tol(oracle.error_weight(wg.wq, wg.scales, wg.biases, xs), wg.K, order="decode")
    assert np.all(np.abs(host_f64(g) - y64) <= T)
    qkvg64 = np.concatenate([oracle.matmul_rows(c2g["qkv"].wq, c2g["qkv"].scales, c2g["qkv"].biases, xs), y64], axis=1)
    assert np.array_equal(oracle.attention_gate(qkvg64, NQ, NKV, NG), y64)



@pytest.mark.parametrize("fused", [False, True])
def test_rows_at_the_same_position_keep_separate_rings(c2, fused):
    """Rows of separate streams at one position (equal ring slots) write
    rings of their own ([rows][ring][kv][64] caches): each row's ring equals
    that row's one-row call, and the other slots stay untouched."""
    case = CASES[1]
    R = 4
    pos_np = np.array([7, 7, 7 + RING, 300], dtype=np.int32)  # rows 0..2 share slot 7
    say(f"per-row rings, equal slots, fused={fused}")
    gq, gk = _gammas(c2, case)
    w = c2["qkv"]

    def call(rows, pos, k, v):
        q = torch.full((len(rows), NQ * 64), float("nan"), device=DEV)
        xr = c2["xd"][rows[0] : rows[-1] + 1]
        if fused:
            q4.qmv_qkv_rope(c2["p"], w.K, xr, pos, NQ, NKV, case["rot"], case["theta"], q, k, v, gq, gk)
        else:
            y = q4.qmv_rows(c2["p"], w.N, w.K, xr)
            q4.rope_kv_store(y, pos, NQ, NKV, case["rot"], case["theta"], q, k, v, gq, gk)
        return q

    k = torch.full((R, RING, NKV, 64), float("nan"), device=DEV)
    v = torch.full((R, RING, NKV, 64), float("nan"), device=DEV)
    q = call(list(range(R)), torch.from_numpy(pos_np).to(DEV), k, v)
    torch.cuda.synchronize()
    for r in range(R):
        k1 = torch.full((RING, NKV, 64), float("nan"), device=DEV)
        v1 = torch.full((RING, NKV, 64), float("nan"), device=DEV)
        q1 = call([r], torch.from_numpy(pos_np[r : r + 1]).to(DEV), k1, v1)
        torch.cuda.synchronize()
        assert np.array_equal(bits32(q1)[0], bits32(q)[r])
        assert np.array_equal(bits32(k1), bits32(k[r])), r
        assert np.array_equal(bits32(v1), bits32(v[r])), r
        slot = int(pos_np[r]) % RING
        written = torch.zeros(RING, dtype=torch.bool)
        written[slot] = True
        assert torch.isnan(k[r][~written]).all() and not torch.isnan(k[r][slot]).any()
