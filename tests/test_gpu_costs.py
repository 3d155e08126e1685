"""Window-cost table (TensorFold PR #1696, later revision, "What it adds" >
Exact speed work: costs measured at load at five row counts from 1 to 16,
interpolated in between) on the GPU: five
positive timings, the interpolation reads them back at the timed row counts,
and the timed launches compute the same bits as a plain call."""

import math

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import synthetic
from tests.gpu_helpers import bits32, dev_bf16, dev_f32, dev_weight, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("bits,xf32", [(4, False), (4, True), (8, False)])
def test_window_costs_table(bits, xf32):
    rng = np.random.default_rng(900 + bits)
    w = synthetic.draw_qweight(rng, "w", 3072, 2048, bits=bits)
    p = dev_weight(w)
    x = dev_f32(synthetic.draw_f32_rows(rng, 16, 2048)) if xf32 else dev_bf16(synthetic.draw_bf16_rows(rng, 16, 2048))
    y = torch.empty((16, 3072), dtype=torch.float32, device="cuda:0")
    costs = q4.window_costs(p, w.N, w.K, x, bits=bits, reps=20, y=y)
    say(f"window costs bits={bits} f32={xf32}: " + ", ".join(f"{c:.2f}" for c in costs))
    assert len(costs) == 5 and all(math.isfinite(c) and 0.0 < c < 1e4 for c in costs)
    for R, c in zip(q4.WINDOW_COST_ROWS, costs):
        assert q4.window_cost(costs, R) == c
    # the last timed launches ran R = 16: y holds their result
    ref = q4.qmv_rows(p, w.N, w.K, x, bits=bits)
    torch.cuda.synchronize()
    assert np.array_equal(bits32(y), bits32(ref))
