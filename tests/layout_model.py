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
