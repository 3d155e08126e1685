"""A numpy model of the packed device layout documented in include/q4g64.h,
written from that description (test code; shares nothing with the kernels).
Used to check the pack kernel bit for bit."""

import numpy as np

# position of code e (k offset e within 8) inside a device word
DEV_NIBBLE = [0, 2, 4, 6, 1, 3, 5, 7]


def packed_bytes(N, K):
    return (N // 16) * ((K // 64 + 1) // 2) * 1152


def pack_model(wq, scales, biases, N, K):
    T, G = N // 16, K // 64
    P = (G + 1) // 2
    wq = np.asarray(wq, dtype=np.uint32)
    t = np.arange(T)[:, None, None, None]
    p = np.arange(P)[None, :, None, None]
    L = np.arange(64)[None, None, :, None]
    h = np.arange(4)[None, None, None, :]
    n = 16 * t + L % 16
    kb = 128 * p + 32 * h + 8 * (L // 16)
    n, kb = np.broadcast_arrays(n, kb)
    valid = kb < K
    cw = wq[n, np.where(valid, kb // 8, 0)]
    dev = np.zeros(valid.shape, dtype=np.uint32)
    for e in range(8):
        dev |= ((cw >> np.uint32(4 * e)) & np.uint32(0xF)) << np.uint32(4 * DEV_NIBBLE[e])
    dev = np.where(valid, dev, 0).astype(np.uint32)
    sc = np.asarray(scales, dtype=np.uint32)
    bi = np.asarray(biases, dtype=np.uint32)
    sb = np.zeros((T, P, 16, 2), dtype=np.uint32)
    for j in range(2):
        g = 2 * np.arange(P) + j
        ok = g < G
        gg = np.where(ok, g, 0)
        cols = 16 * np.arange(T)[:, None, None] + np.arange(16)[None, None, :]
        word = sc[cols, gg[None, :, None]] | (bi[cols, gg[None, :, None]] << np.uint32(16))
        sb[:, :, :, j] = np.where(ok[None, :, None], word, 0)
    return np.concatenate([dev.reshape(-1).view(np.uint8), sb.reshape(-1).view(np.uint8)])


def packed_bytes_bits(N, K, bits):
    return (N // 16) * ((K // 64 + 1) // 2) * (256 * bits + 128)


def pack_model_bits(codes, scales, biases, N, K, bits):
    """Packed layout for 6- or 8-bit codes, from the header's description.
    ``codes`` is the [N][K] array of code values (unpacked canonical input)."""
    T, G = N // 16, K // 64
    P = (G + 1) // 2
    q = np.zeros((N, P * 128), dtype=np.uint32)
    q[:, :K] = np.asarray(codes, dtype=np.uint32)

    def half_codes(t, p, L, h):
        """codes e = 0..7 of column 16t + L%16 at k = 128p + 32h + 8(L//16) + e"""
        n = 16 * t + L % 16
        k0 = 128 * p + 32 * h + 8 * (L // 16)
        return q[n, k0 : k0 + 8]

    blocks = []
    for t in range(T):
        for p in range(P):
            if bits == 8:
                words = np.zeros((2, 64, 4), dtype=np.uint32)
                for j in range(2):
                    for L in range(64):
                        for hh in range(2):
                            c = half_codes(t, p, L, 2 * j + hh)
                            words[j, L, 2 * hh] = c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24
                            words[j, L, 2 * hh + 1] = c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24
                blocks.append(words.reshape(-1))
            else:
                low = np.zeros((64, 4), dtype=np.uint32)
                high = np.zeros((64, 2), dtype=np.uint32)
                for L in range(64):
                    for h in range(4):
                        c = half_codes(t, p, L, h)
                        for e in range(8):
                            low[L, h] |= (c[e] & 0xF) << (4 * DEV_NIBBLE[e])
                    for j in range(2):
                        for hh in range(2):
                            c = half_codes(t, p, L, 2 * j + hh)
                            for b in range(4):
                                high[L, j] |= (c[b] >> 4) << (8 * b + 4 * hh)
                                high[L, j] |= (c[4 + b] >> 4) << (8 * b + 4 * hh + 2)
                blocks.append(np.concatenate([low.reshape(-1), high.reshape(-1)]))
    dev = np.concatenate(blocks).astype(np.uint32)
    sb_part = pack_model(np.zeros((N, K // 8), dtype=np.uint32), scales, biases, N, K)[(N // 16) * P * 1024 :]
    return np.concatenate([dev.view(np.uint8), sb_part])


def pack_model_fp8(w8, scales, N, K):
    """Packed layout of block-FP8 weights, from the header: the E4M3 bytes in
    the 8-bit code layout, then for column n of pair p both words set to the
    float32 scale of block (n // 128, p) (the second zero past G)."""
    T, G = N // 16, K // 64
    P = (G + 1) // 2
    codes = pack_model_bits(np.asarray(w8, dtype=np.uint8), np.zeros((N, G), np.uint16), np.zeros((N, G), np.uint16), N, K, 8)
    codes = codes[: T * P * 2048]
    s = np.asarray(scales, dtype=np.float32).view(np.uint32)
    sb = np.zeros((T, P, 16, 2), dtype=np.uint32)
    for t in range(T):
        for p in range(P):
            for c in range(16):
                v = s[(16 * t + c) // 128, p]
                sb[t, p, c, 0] = v
                sb[t, p, c, 1] = v if 2 * p + 1 < G else 0
    return np.concatenate([codes, sb.reshape(-1).view(np.uint8)])
