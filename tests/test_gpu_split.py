"""The decode matvec with K split over several workgroups per column tile
(qmv_rows_split): bit-identical to qmv_rows for every split count, every
activation form and code width; the workspace's counters return to zero;
consecutive calls with new inputs on one workspace never see an earlier
call's partials; and the results sit within the decode tolerance of the
float64 oracle."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import synthetic
from tests.gpu_helpers import DEV, bits32, check_within, dev_bf16, dev_f32, dev_weight, host_f64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mats():
    d1 = synthetic.config(1)
    d2 = synthetic.config(2)
    out = {"w2": d1["w2"], "qkv": synthetic.concat_rows(d2["wq"], d2["wk"], d2["wv"], name="qkv"), "wo": d2["wo"]}
    for k in list(out):
        out["p_" + k] = dev_weight(out[k])
    rng = np.random.default_rng(77)
    out["xf"] = synthetic.draw_f32_rows(rng, 16, 8192, sigma=0.05)
    out["xb"] = d2["x"]
    return out


def _work(N, K, xdt, R, splits, bits=4):
    nb = q4.split_work_bytes(N, K, xdt, R, splits, bits=bits)
    assert nb > 0
    return q4.split_workspace(nb, DEV)


def _counters_zero(work, N):
    # a 32-bit counter per tile id at the start of the workspace (at least N / 16 of them)
    return int(work[: 4 * (N // 16)].view(torch.int32).abs().sum().item()) == 0


@pytest.mark.parametrize("R", [1, 2, 5, 16])
@pytest.mark.parametrize("splits", [0, 2, 4, 16])
def test_w2_float32_rows_split_equals_unsplit(mats, R, splits):
    w = mats["w2"]
    say(f"qmv_rows_split w2 {w.N}x{w.K} f32 R={R} splits={splits}")
    x = dev_f32(mats["xf"][:R])
    ref = q4.qmv_rows(mats["p_w2"], w.N, w.K, x)
    work = _work(w.N, w.K, q4.Q4_F32, R, splits)
    y = q4.qmv_rows_split(mats["p_w2"], w.N, w.K, x, work, splits=splits)
    torch.cuda.synchronize()
    assert np.array_equal(bits32(y), bits32(ref))
    assert _counters_zero(work, w.N)


@pytest.mark.parametrize("R", [1, 4, 16])
def test_w2_planes_split_equals_unsplit(mats, R):
    w = mats["w2"]
    say(f"qmv_rows_split w2 planes R={R}")
    xf = mats["xf"][:R]
    # the three exact bf16 pieces, as the fused gate writes them
    z3 = torch.empty((3, R, w.K), dtype=torch.bfloat16, device=DEV)
    zt = q4.TiledPlanes.empty(R, w.K, DEV)
    d1 = synthetic.config(1)
    # planes of the SwiGLU output of the workload's w1/w3 for these rows' stand-in
    p1, p3 = dev_weight(d1["w1"]), dev_weight(d1["w3"])
    xb = dev_bf16(mats["xb"][:R])
    q4.qmv_w13_swiglu(p1, p3, d1["w1"].N, d1["w1"].K, xb, y=z3, planes=True)
    q4.qmv_w13_swiglu(p1, p3, d1["w1"].N, d1["w1"].K, xb, y=zt, planes="tiled")
    for xin, xdt in ((z3, q4.Q4_BF16X3), (zt, q4.Q4_BF16X3T)):
        ref = q4.qmv_rows(mats["p_w2"], w.N, w.K, xin)
        work = _work(w.N, w.K, xdt, R, 0)
        y = q4.qmv_rows_split(mats["p_w2"], w.N, w.K, xin, work)
        torch.cuda.synchronize()
        assert np.array_equal(bits32(y), bits32(ref)), xdt
        assert _counters_zero(work, w.N)
    del xf


@pytest.mark.parametrize("name", ["qkv", "wo"])
@pytest.mark.parametrize("R", [1, 3, 16])
@pytest.mark.parametrize("splits", [0, 2, 8])
def test_attention_projections_split_equals_unsplit(mats, name, R, splits):
    w = mats[name]
    say(f"qmv_rows_split {name} {w.N}x{w.K} bf16 R={R} splits={splits}")
    x = dev_bf16(mats["xb"][:R])
    ref = q4.qmv_rows(mats["p_" + name], w.N, w.K, x)
    work = _work(w.N, w.K, q4.Q4_BF16, R, splits)
    y = q4.qmv_rows_split(mats["p_" + name], w.N, w.K, x, work, splits=splits)
    torch.cuda.synchronize()
    assert np.array_equal(bits32(y), bits32(ref))
    assert _counters_zero(work, w.N)


def test_new_inputs_on_one_workspace(mats):
    """Six calls in a row on one workspace, each with new activations (and
    two row counts): every result equals its unsplit call, so no call reads
    partials an earlier call left behind."""
    w = mats["w2"]
    say("qmv_rows_split: consecutive calls with new inputs on one workspace")
    work = _work(w.N, w.K, q4.Q4_F32, 16, 2)
    rng = np.random.default_rng(5)
    outs, refs = [], []
    for c in range(6):
        R = 1 if c % 2 == 0 else 7
        x = dev_f32(synthetic.draw_f32_rows(rng, R, w.K, sigma=0.05))
        outs.append(q4.qmv_rows_split(mats["p_w2"], w.N, w.K, x, work, splits=2))
        refs.append(q4.qmv_rows(mats["p_w2"], w.N, w.K, x))
    torch.cuda.synchronize()
    for a, b in zip(outs, refs):
        assert np.array_equal(bits32(a), bits32(b))
    assert _counters_zero(work, w.N)


@pytest.mark.parametrize("bits", [4, 6, 8])
@pytest.mark.parametrize("N,K,R", [(64, 64, 1), (192, 320, 3), (320, 1344, 16), (128, 4160, 2)])
def test_edge_shapes_and_widths(N, K, R, bits):
    say(f"qmv_rows_split edge N={N} K={K} R={R} bits={bits}")
    rng = np.random.default_rng(N + K + R + bits)
    w = synthetic.draw_qweight(rng, "e", N, K, bits=bits)
    p = dev_weight(w)
    x = synthetic.draw_bf16_rows(rng, R, K)
    xf = synthetic.draw_f32_rows(rng, R, K, sigma=0.5)
    for xin, xdt, xh in ((dev_bf16(x), q4.Q4_BF16, x), (dev_f32(xf), q4.Q4_F32, xf)):
        ref = q4.qmv_rows(p, N, K, xin, bits=bits)
        for splits in (0, 3, 16):
            nb = q4.split_work_bytes(N, K, xdt, R, splits, bits=bits)
            work = q4.split_workspace(nb, DEV)
            y = q4.qmv_rows_split(p, N, K, xin, work, splits=splits, bits=bits)
            torch.cuda.synchronize()
            assert np.array_equal(bits32(y), bits32(ref)), (xdt, splits)
        check_within(host_f64(y), w, xh, x_dtype="bf16" if xdt == q4.Q4_BF16 else "f32", label=f"split edge {N}x{K}",
                     order="decode")


def test_split_within_tolerance_of_the_oracle(mats):
    w = mats["w2"]
    say("qmv_rows_split w2 f32 R=3 against the float64 oracle")
    x = mats["xf"][:3]
    work = _work(w.N, w.K, q4.Q4_F32, 3, 0)
    y = q4.qmv_rows_split(mats["p_w2"], w.N, w.K, dev_f32(x), work)
    torch.cuda.synchronize()
    cols = np.arange(0, w.N, 3)
    check_within(host_f64(y)[:, cols], w, x, cols=cols, x_dtype="f32", label="split w2", order="decode")
