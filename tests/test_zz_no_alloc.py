"""qmv_rows_split_noalloc, the split decode matvec for callers that cannot
allocate: called through the C ABI, its output must equal the existing
qmv_rows_split (caller workspace) bit for bit, on two calls in a row, the
second with a smaller input, and must leave the library's scratch counters
ready for the next call."""

import ctypes

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import synthetic
from tests.gpu_helpers import DEV, bits32, dev_f32, dev_weight, say

pytestmark = pytest.mark.gpu


def _noalloc(p, N, K, x, xdt, ldx, R, y, splits):
    lib = q4.lib()
    rc = lib.qmv_rows_split_noalloc(4, p.data_ptr(), N, K, x.data_ptr(), xdt, ldx, R, y.data_ptr(), y.stride(0), splits,
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == q4.Q4_OK, lib.q4_last_error().decode()


def test_noalloc_equals_the_workspace_call_twice_in_a_row():
    d = synthetic.config(1)
    w = d["w2"]
    p = dev_weight(w)
    rng = np.random.default_rng(123)
    assert q4.lib().qmv_split_noalloc_max_bytes() == 8 << 20
    # first call: 16 float32 rows; second: 1 row (a smaller input)
    for R, splits in ((16, 2), (1, 0)):
        say(f"qmv_rows_split_noalloc w2 {w.N}x{w.K} f32 R={R} splits={splits}")
        xh = synthetic.draw_f32_rows(rng, R, w.K, sigma=0.05)
        x = dev_f32(xh)
        y = torch.full((R, w.N), float("nan"), device=DEV)
        _noalloc(p, w.N, w.K, x, q4.Q4_F32, w.K, R, y, splits)
        work = q4.split_workspace(q4.split_work_bytes(w.N, w.K, q4.Q4_F32, R, splits), DEV)
        ref = q4.qmv_rows_split(p, w.N, w.K, x, work, splits=splits)
        torch.cuda.synchronize()
        assert np.array_equal(bits32(y), bits32(ref)), R
        assert np.array_equal(bits32(y), bits32(q4.qmv_rows(p, w.N, w.K, x))), R


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    # 65536 columns x 16 segments x 16 bf16 rows split 2 ways needs 64 MiB of partials
    lib = q4.lib()
    fake = 0x10000
    rc = lib.qmv_rows_split_noalloc(4, fake, 65536, 4096, fake, q4.Q4_BF16, 4096, 16, fake, 65536, 2, None)
    assert rc == q4.Q4_EUNSUPPORTED
    assert "scratch" in lib.q4_last_error().decode()
