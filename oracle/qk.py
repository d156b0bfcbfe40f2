"""q/k head norm, half-split RoPE and the K/V append of one attention layer
over every row of a shared round (oracle; test infrastructure only).

PR #1377 "LFM2: shared-round decode": per stream an attention layer is a qk
launch, the attention and the merge (the shared-round commit counts 10 such
layers a forward beside 30 conv layers; the inline-bodies commit names the
qk row body); the shared round runs each of them once a layer over every row
through the table of the streams' cache addresses, row offsets and key
counts. PR #1391 "lfm2: draft with LiquidAI's DSpark drafter (--drafter)":
the target's RoPE kernel is half-split (the drafter's q and k rows and their
norm gains are reordered so that it gives the drafter's interleaved RoPE),
and the config admission is asked to refuse a rope theta that is not a
finite positive number.

The pages print no formula for the stage; the readings taken (listed in the
design notes) are:

* a row's qkv projection is bf16 [3072] = q (32 heads x 64) | k (8 x 64) |
  v (8 x 64);
* each q and k head is RMS-normed over its 64 values with a 64-wide gain
  shared by the heads (the pages speak of norm gains, no bias):
  y = x / sqrt(mean(x^2) + eps) * g;
* half-split RoPE at key position pos: for i < 32, a_i = pos * theta^(-i/32)
  and (y_i, y_{i+32}) -> (y_i cos a_i - y_{i+32} sin a_i,
  y_{i+32} cos a_i + y_i sin a_i);
* row p of stream s (w_s rows, K_s keys counting the window) sits at key
  position K_s - w_s + p, the keys its K and V are appended at;
* q goes to Q [rows][32][64]; k and v go to the stream's cache at that
  position, every other cache entry untouched; each output value is rounded
  to bf16 once (nearest, ties to even); v is copied exactly;
* theta and eps are parameters (not on the pages).
"""

import numpy as np

from . import bf16

N_Q, N_KV, D = 32, 8, 64
QKV = (N_Q + 2 * N_KV) * D


def positions(streams):
    """(stream, key position) of every row, streams in caller order."""
    st, pos = [], []
    for s, (w, K, _cap) in enumerate(streams):
        for p in range(int(w)):
            st.append(s)
            pos.append(int(K) - int(w) + p)
    return np.array(st, dtype=np.int64), np.array(pos, dtype=np.int64)


def norm_rope(x, gain, pos, theta, eps):
    """x: float64 [H][64] heads of one row; gain: float64 [64]. Returns the
    normed and rotated heads, float64, unrounded."""
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(gain, dtype=np.float64)
    a = float(pos) * np.power(float(theta), -np.arange(D // 2, dtype=np.float64) / (D // 2))
    c, s = np.cos(a), np.sin(a)
    lo, hi = y[..., :D // 2], y[..., D // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def qk_rows(streams, qkv, q_gain, k_gain, theta, eps):
    """qkv: uint16 [rows][3072]; gains uint16 [64]. Returns (Q [rows][32][64],
    K_new [rows][8][64], V_new [rows][8][64]) as bf16 bits, plus the rows'
    streams and key positions."""
    qkv = np.asarray(qkv, dtype=np.uint16)
    st, pos = positions(streams)
    R = len(st)
    assert qkv.shape == (R, QKV)
    gq, gk = bf16.to_f64(q_gain), bf16.to_f64(k_gain)
    Q = np.zeros((R, N_Q, D), dtype=np.uint16)
    Kn = np.zeros((R, N_KV, D), dtype=np.uint16)
    Vn = np.zeros((R, N_KV, D), dtype=np.uint16)
    for r in range(R):
        row = qkv[r]
        q = bf16.to_f64(row[:N_Q * D]).reshape(N_Q, D)
        k = bf16.to_f64(row[N_Q * D:(N_Q + N_KV) * D]).reshape(N_KV, D)
        Q[r] = bf16.round_f64(norm_rope(q, gq, pos[r], theta, eps))
        Kn[r] = bf16.round_f64(norm_rope(k, gk, pos[r], theta, eps))
        Vn[r] = row[(N_Q + N_KV) * D:].reshape(N_KV, D)
    return Q, Kn, Vn, st, pos


def append(K_list, V_list, st, pos, Kn, Vn):
    """Copies of the streams' logical caches ([8][cap][64] bf16 bits) with
    every row's k and v written at its key position."""
    K_out = [np.array(k, dtype=np.uint16, copy=True) for k in K_list]
    V_out = [np.array(v, dtype=np.uint16, copy=True) for v in V_list]
    for r in range(len(st)):
        K_out[st[r]][:, pos[r], :] = Kn[r]
        V_out[st[r]][:, pos[r], :] = Vn[r]
    return K_out, V_out
