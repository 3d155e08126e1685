"""Plain float64 oracle for the attention-side decode epilogue: QK norm,
partial RoPE and the KV store applied to the q/k/v matvec output.

TEST INFRASTRUCTURE (see ``oracle/__init__``); it shares no code with the
HIP path.

What it computes (TensorFold PR #1696, "What it adds": the LFM3 kernels
include QK norm with partial RoPE and GQA attention over a KV ring; decode
fuses RoPE with the KV store). The pages give neither formulas nor
constants; the readings, all parameters of the call:

* The stacked matvec output of one row is [q heads | k heads | v heads],
  head_dim = 64 each (the workload's 32 q and 8 kv heads).
* QK norm (optional): per head, x <- x / sqrt(mean(x^2) + eps) * gamma,
  gamma one 64-vector for all q heads and one for all k heads.
* Partial RoPE on q and k: the first ``rot`` dims of a head (rot even) are
  rotated in half-split pairs (i, i + rot/2), i < rot/2, by the angle
  pos * theta^(-2i/rot); the remaining dims pass through. v is not rotated.
* KV store: the row's k and v heads are written at slot pos mod ring of a
  [ring][kv_heads][64] cache; q is returned.
"""

from __future__ import annotations

import numpy as np

HEAD = 64


def rms_norm(x: np.ndarray, gamma, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def rope_angles(pos, rot: int, theta: float) -> np.ndarray:
    """[len(pos)][rot/2] angles pos * theta^(-2i/rot), float64."""
    i = np.arange(rot // 2, dtype=np.float64)
    inv = np.power(float(theta), -2.0 * i / rot)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def rope(x: np.ndarray, pos, rot: int, theta: float) -> np.ndarray:
    """Half-split rotation of the first ``rot`` dims of every head.
    x: [rows][heads][64]; pos: [rows]."""
    x = np.array(x, dtype=np.float64)
    if rot == 0:
        return x
    h = rot // 2
    a = rope_angles(pos, rot, theta)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :h].copy(), x[..., h:rot].copy()
    x[..., :h] = x1 * c - x2 * s
    x[..., h:rot] = x2 * c + x1 * s
    return x


def rope_kv(qkv, pos, n_q: int, n_kv: int, rot: int, theta: float, gamma_q=None, gamma_k=None, eps: float = 1e-6):
    """The epilogue on float64 rows qkv [R][(n_q + 2 n_kv) * 64]. Returns
    (q [R][n_q*64], k [R][n_kv][64], v [R][n_kv][64]) in float64; the caller
    places k and v at slots pos mod ring."""
    qkv = np.asarray(qkv, dtype=np.float64)
    R = qkv.shape[0]
    q = qkv[:, : n_q * HEAD].reshape(R, n_q, HEAD)
    k = qkv[:, n_q * HEAD : (n_q + n_kv) * HEAD].reshape(R, n_kv, HEAD)
    v = qkv[:, (n_q + n_kv) * HEAD : (n_q + 2 * n_kv) * HEAD].reshape(R, n_kv, HEAD)
    if gamma_q is not None:
        q = rms_norm(q, gamma_q, eps)
    if gamma_k is not None:
        k = rms_norm(k, gamma_k, eps)
    return rope(q, pos, rot, theta).reshape(R, n_q * HEAD), rope(k, pos, rot, theta), v.copy()


def attention_gate(qkvg, n_q: int, n_kv: int, n_gate: int) -> np.ndarray:
    """The gate heads stacked after v (gated attention's fourth matvec), [R][n_gate * 64] float64: the epilogue passes
    them through unchanged, since the gate acts inside attention."""
    qkvg = np.asarray(qkvg, dtype=np.float64)
    lo = (n_q + 2 * n_kv) * HEAD
    return qkvg[:, lo : lo + n_gate * HEAD].copy()
