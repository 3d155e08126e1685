"""The decode FFN step (qmv_ffn) on the GPU: one launch up to 2 rows, two
launches (z handed over as fragment-ordered planes in the workspace) from 3.

It must return exactly the bits of the two-call composition
qmv_w13_swiglu -> qmv_rows (float32 input), whose parity with the float64
oracle the decode tests establish; every row must equal its one-row result;
the workspace's state must survive repeated calls, changing row counts and
graph replays; and its error word must stay 0."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import oracle
import synthetic
from tests.gpu_helpers import DEV, bits32, dev_bf16, dev_weight, host_f64, say
from tests.tolerance import tol, tol_swiglu

pytestmark = pytest.mark.gpu


def _composed(p1, p3, p2, N1, K1, N2, x):
    z = q4.qmv_w13_swiglu(p1, p3, N1, K1, x)
    y = q4.qmv_rows(p2, N2, N1, z)
    return z, y


def _weights(seed, N1, K1, N2):
    rng = np.random.default_rng(seed)
    w1 = synthetic.draw_qweight(rng, "w1", N1, K1)
    w3 = synthetic.draw_qweight(rng, "w3", N1, K1)
    w2 = synthetic.draw_qweight(rng, "w2", N2, N1)
    return rng, w1, w3, w2


@pytest.fixture(scope="module")
def c1():
    d = synthetic.config(1)
    d["p1"], d["p3"], d["p2"] = dev_weight(d["w1"]), dev_weight(d["w3"]), dev_weight(d["w2"])
    return d


def test_c1_step_equals_composition_and_oracle(c1):
    w1, w2 = c1["w1"], c1["w2"]
    N1, K1, N2 = w1.N, w1.K, w2.N
    say(f"qmv_ffn c1 N1={N1} K1={K1} N2={N2} R=1")
    x = dev_bf16(c1["x"])
    work = q4.ffn_workspace(N1, N2, 1, DEV)
    z, y = q4.qmv_ffn(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x, work)
    zc, yc = _composed(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x)
    torch.cuda.synchronize()
    assert q4.ffn_error(work) == 0
    assert np.array_equal(bits32(z), bits32(zc))
    assert np.array_equal(bits32(y), bits32(yc))
    # and the chain against the oracle's float64 chain, with the propagated bound
    w3 = c1["w3"]
    a64 = oracle.matmul_rows(w1.wq, w1.scales, w1.biases, c1["x"])
    c64 = oracle.matmul_rows(w3.wq, w3.scales, w3.biases, c1["x"])
    z64 = oracle.swiglu(a64, c64)
    Tz = tol_swiglu(a64, c64, tol(oracle.error_weight(w1.wq, w1.scales, w1.biases, c1["x"]), K1, order="decode"),
                    tol(oracle.error_weight(w3.wq, w3.scales, w3.biases, c1["x"]), K1, order="decode"))
    assert np.all(np.abs(host_f64(z) - z64) <= Tz)
    y64 = oracle.matmul_rows(w2.wq, w2.scales, w2.biases, z64)
    bound = tol(oracle.error_weight(w2.wq, w2.scales, w2.biases, np.abs(z64) + Tz), w2.K, "f32", order="decode") + \
        oracle.error_weight(w2.wq, w2.scales, w2.biases, Tz)
    ratio = float(np.max(np.abs(host_f64(y) - y64) / bound))
    say(f"qmv_ffn c1 y max err/bound {ratio:.3g}")
    assert ratio <= 1.0


@pytest.mark.parametrize("R", [2, 3, 5, 16])
def test_rows_equal_composition_and_one_row(c1, R):
    w1, w2 = c1["w1"], c1["w2"]
    N1, K1, N2 = w1.N, w1.K, w2.N
    say(f"qmv_ffn c1 shapes R={R}")
    rng = np.random.default_rng(100 + R)
    xb = synthetic.draw_bf16_rows(rng, R, K1)
    x = dev_bf16(xb)
    work = q4.ffn_workspace(N1, N2, R, DEV)
    z, y = q4.qmv_ffn(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x, work)
    zc, yc = _composed(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x)
    torch.cuda.synchronize()
    assert q4.ffn_error(work) == 0
    assert np.array_equal(bits32(z), bits32(zc))
    assert np.array_equal(bits32(y), bits32(yc))
    for r in (0, R - 1):
        z1, y1 = q4.qmv_ffn(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x[r : r + 1], work)
        torch.cuda.synchronize()
        assert np.array_equal(bits32(z1)[0], bits32(z)[r])
        assert np.array_equal(bits32(y1)[0], bits32(y)[r])


@pytest.mark.parametrize("R", [1, 5])
def test_repeated_calls_reuse_the_workspace(c1, R):
    """Five calls on one workspace: one row runs the one-launch step (its call
    counter advances once per call), five rows the two calls (which leave the
    counter alone)."""
    w1, w2 = c1["w1"], c1["w2"]
    N1, K1, N2 = w1.N, w1.K, w2.N
    say(f"qmv_ffn c1 five calls on one workspace R={R}")
    x = dev_bf16(synthetic.draw_bf16_rows(np.random.default_rng(3), R, K1))
    work = q4.ffn_workspace(N1, N2, R, DEV)
    ref = None
    for _ in range(5):
        z, y = q4.qmv_ffn(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x, work)
        torch.cuda.synchronize()
        cur = (bits32(z), bits32(y))
        if ref is None:
            ref = cur
        assert np.array_equal(cur[0], ref[0]) and np.array_equal(cur[1], ref[1])
    state = work.view(torch.int32).cpu().numpy()
    assert state[q4.FFN_ERR_OFFSET // 4] == 0
    assert state[q4.FFN_FLOW_EPOCH_OFFSET // 4] == (5 if R == 1 else 0)


def test_new_inputs_each_call_on_one_workspace(c1):
    """Eight calls in a row on one workspace, each with new activations and
    row counts 1..4 and 7 (the one-launch and the two-call step in turn): every
    result equals the composition of the two decode calls, so no call reads
    values an earlier call left in the workspace."""
    w1, w2 = c1["w1"], c1["w2"]
    N1, K1, N2 = w1.N, w1.K, w2.N
    say("qmv_ffn c1: eight calls with new inputs on one workspace")
    work = q4.ffn_workspace(N1, N2, 4, DEV)
    rng = np.random.default_rng(8)
    for R in (1, 2, 1, 4, 7, 3, 1, 1):
        x = dev_bf16(synthetic.draw_bf16_rows(rng, R, K1))
        z, y = q4.qmv_ffn(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x, work)
        zc, yc = _composed(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x)
        torch.cuda.synchronize()
        assert q4.ffn_error(work) == 0
        assert np.array_equal(bits32(z), bits32(zc)), R
        assert np.array_equal(bits32(y), bits32(yc)), R


@pytest.mark.parametrize("N1,K1,N2,R", [(64, 64, 64, 1), (192, 128, 128, 3), (8192, 2048, 4096, 1), (8192, 4096, 2048, 2),
                                        (4096, 2048, 1024, 16), (512, 256, 64, 4), (256, 2048, 2048, 1), (1024, 512, 8192, 3),
                                        (7936, 1280, 192, 2)])
def test_shapes_equal_composition(N1, K1, N2, R):
    say(f"qmv_ffn N1={N1} K1={K1} N2={N2} R={R}")
    rng, w1, w3, w2 = _weights(7 + N1 + K1, N1, K1, N2)
    p1, p3, p2 = dev_weight(w1), dev_weight(w3), dev_weight(w2)
    x = dev_bf16(synthetic.draw_bf16_rows(rng, R, K1))
    work = q4.ffn_workspace(N1, N2, R, DEV)
    z, y = q4.qmv_ffn(p1, p3, p2, N1, K1, N2, x, work)
    zc, yc = _composed(p1, p3, p2, N1, K1, N2, x)
    torch.cuda.synchronize()
    assert q4.ffn_error(work) == 0
    assert np.array_equal(bits32(z), bits32(zc))
    assert np.array_equal(bits32(y), bits32(yc))


@pytest.mark.parametrize("R", [1, 4])
def test_graph_replays_equal_eager(c1, R):
    """One row: the one-launch step; four rows: the two launches."""
    w1, w2 = c1["w1"], c1["w2"]
    N1, K1, N2 = w1.N, w1.K, w2.N
    say(f"qmv_ffn c1 in a HIP graph, four replays, R={R}")
    x = dev_bf16(c1["x"] if R == 1 else synthetic.draw_bf16_rows(np.random.default_rng(11), R, K1))
    work = q4.ffn_workspace(N1, N2, R, DEV)
    z = torch.empty((R, N1), dtype=torch.float32, device=DEV)
    y = torch.empty((R, N2), dtype=torch.float32, device=DEV)
    z_ref, y_ref = q4.qmv_ffn(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x, work)
    torch.cuda.synchronize()
    zr, yr = bits32(z_ref), bits32(y_ref)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            q4.qmv_ffn(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x, work, z=z, y=y)
    torch.cuda.synchronize()
    for k in range(4):
        z.zero_()
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits32(z), zr), k
        assert np.array_equal(bits32(y), yr), k
        # eager work between replays
        q4.qmv_ffn(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x, work)
        torch.cuda.synchronize()
    assert q4.ffn_error(work) == 0


@pytest.mark.parametrize("R", [2, 6])
def test_padded_outputs_keep_their_padding(c1, R):
    """z and y as views of wider buffers (row strides N + 64): the rows hold
    the composition's bits and the padding is untouched, on the one-launch
    step (2 rows) and the two launches (6 rows)."""
    w1, w2 = c1["w1"], c1["w2"]
    N1, K1, N2 = w1.N, w1.K, w2.N
    say(f"qmv_ffn c1 padded z and y, R={R}")
    x = dev_bf16(synthetic.draw_bf16_rows(np.random.default_rng(21 + R), R, K1))
    work = q4.ffn_workspace(N1, N2, R, DEV)
    zbuf = torch.full((R, N1 + 64), -7.0, dtype=torch.float32, device=DEV)
    ybuf = torch.full((R, N2 + 64), -7.0, dtype=torch.float32, device=DEV)
    q4.qmv_ffn(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x, work, z=zbuf[:, :N1], y=ybuf[:, :N2])
    zc, yc = _composed(c1["p1"], c1["p3"], c1["p2"], N1, K1, N2, x)
    torch.cuda.synchronize()
    assert q4.ffn_error(work) == 0
    assert np.array_equal(bits32(zbuf[:, :N1]), bits32(zc))
    assert np.array_equal(bits32(ybuf[:, :N2]), bits32(yc))
    assert torch.all(zbuf[:, N1:] == -7.0) and torch.all(ybuf[:, N2:] == -7.0)
