"""pack_q4g64 is an integer permutation: bit-exact against the layout model
written from the header, and unpack inverts it."""

import numpy as np
import pytest
import torch

import bit_weight_only_q4g64_amd as q4
import synthetic
from tests.gpu_helpers import DEV, dev_weight, say
from tests.layout_model import pack_model

pytestmark = pytest.mark.gpu


def _weights():
    rng = np.random.default_rng(77)
    yield synthetic.config(0)["w"]
    yield synthetic.config(2)["wk"]
    for N, K in ((64, 64), (64, 192), (128, 640), (192, 2048)):
        w = synthetic.draw_qweight(rng, f"r{N}x{K}", N, K)
        # arbitrary 16-bit patterns for scale/bias: pack must not care
        w.scales = rng.integers(0, 1 << 16, w.scales.shape, dtype=np.uint16)
        w.biases = rng.integers(0, 1 << 16, w.biases.shape, dtype=np.uint16)
        yield w


@pytest.mark.parametrize("idx", range(6))
def test_pack_bit_exact_and_invertible(idx):
    w = list(_weights())[idx]
    say(f"pack {w.name} N={w.N} K={w.K}")
    packed = dev_weight(w)
    torch.cuda.synchronize()
    assert packed.numel() == q4.packed_bytes(w.N, w.K)
    model = pack_model(w.wq, w.scales, w.biases, w.N, w.K)
    assert np.array_equal(packed.cpu().numpy(), model)
    wq, sc, bi = q4.unpack(packed, w.N, w.K)
    torch.cuda.synchronize()
    assert np.array_equal(wq.cpu().numpy().view(np.uint32), w.wq)
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), w.scales)
    assert np.array_equal(bi.cpu().numpy().view(np.uint16), w.biases)


def test_pack_deterministic():
    w = synthetic.config(0)["w"]
    a = dev_weight(w)
    b = dev_weight(w)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
