"""The numpy model of the packed layout agrees with the header's description,
checked element by element with plain loops (CPU only)."""

import numpy as np

from tests.layout_model import DEV_NIBBLE, pack_model, packed_bytes
import synthetic


def _locate(buf, N, K, n, k):
    """Code of (n, k) read from the packed bytes by following the header text."""
    G = K // 64
    P = (G + 1) // 2
    t, c = divmod(n, 16)
    p, r = divmod(k, 128)
    h, r = divmod(r, 32)
    kc, e = divmod(r, 8)
    lane = c + 16 * kc
    off = (t * P + p) * 1024 + lane * 16 + h * 4
    word = int.from_bytes(bytes(buf[off : off + 4]), "little")
    return (word >> (4 * DEV_NIBBLE[e])) & 0xF


def _sb(buf, N, K, n, g):
    G = K // 64
    P = (G + 1) // 2
    t, c = divmod(n, 16)
    base = (N // 16) * P * 1024
    off = base + (t * P + g // 2) * 128 + c * 8 + (g % 2) * 4
    word = int.from_bytes(bytes(buf[off : off + 4]), "little")
    return word & 0xFFFF, word >> 16


def test_model_matches_header_description():
    rng = np.random.default_rng(3)
    for N, K in ((32, 192), (16, 64), (48, 384)):
        q = rng.integers(0, 16, (N, K), dtype=np.uint8)
        sc = rng.integers(0, 1 << 16, (N, K // 64), dtype=np.uint16)
        bi = rng.integers(0, 1 << 16, (N, K // 64), dtype=np.uint16)
        buf = pack_model(synthetic.pack_codes_low_nibble_first(q), sc, bi, N, K)
        assert buf.size == packed_bytes(N, K)
        for n in range(N):
            for k in range(K):
                assert _locate(buf, N, K, n, k) == q[n, k]
            for g in range(K // 64):
                assert _sb(buf, N, K, n, g) == (sc[n, g], bi[n, g])
        # padding of an odd group count is zero
        if (K // 64) % 2:
            P = (K // 64 + 1) // 2
            for t in range(N // 16):
                blk = buf[(t * P + P - 1) * 1024 : (t * P + P) * 1024].reshape(64, 4, 4)
                assert not blk[:, 2:, :].any()
