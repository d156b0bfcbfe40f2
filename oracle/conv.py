"""Host replay of the gated short conv (oracle; test infrastructure only).

PR #1377 "LFM2: shared-round decode", shared-round commit: a shared round
runs each conv layer once over every row of every stream, against each
stream's own conv state, and the stream conv is checked against a host
replay of the conv steps. The commit on dense twins names the conv input as
6,144 wide from 2,048-wide rows. The pages do not print the conv's
arithmetic; the readings taken here (listed in the design notes) are:

* a row's 6,144 inputs split as B | C | x, 2,048 channels each;
* bx = bf16(B * x), rounded before it is used and before it enters the state
  (so a window equals a step-by-step replay bit for bit);
* a depthwise causal conv of width 3 over the history
  [state_0, state_1, bx_0, bx_1, ...], tap 0 on the oldest step, no bias:
  y_i = C_i * (W[:,0] h_i + W[:,1] h_{i+1} + W[:,2] h_{i+2});
* the stream's state afterwards is the last two history steps.

Everything is float64 here; only bx is rounded (it is exact in float64, so
its rounding is the single RNE rounding of the true product).
"""

import numpy as np

from . import bf16

HIDDEN = 2048
CONV_IN = 3 * HIDDEN
WIDTH = 3


def replay_stream(X_rows, W, state):
    """Replay one stream's window row by row.

    X_rows: uint16 [w][6144]; W: uint16 [2048][3]; state: uint16 [2][2048].
    Returns (y float64 [w][2048], new_state uint16 [2][2048]).
    """
    X_rows = np.asarray(X_rows, dtype=np.uint16)
    w = X_rows.shape[0]
    Wf = bf16.to_f64(W)
    hist_bits = [np.array(state[0], dtype=np.uint16), np.array(state[1], dtype=np.uint16)]
    y = np.zeros((w, HIDDEN), dtype=np.float64)
    for i in range(w):
        B = bf16.to_f64(X_rows[i, 0:HIDDEN])
        C = bf16.to_f64(X_rows[i, HIDDEN:2 * HIDDEN])
        x = bf16.to_f64(X_rows[i, 2 * HIDDEN:3 * HIDDEN])
        hist_bits.append(bf16.round_f64(B * x))
        conv = np.zeros(HIDDEN, dtype=np.float64)
        for k in range(WIDTH):
            conv += Wf[:, k] * bf16.to_f64(hist_bits[i + k])
        y[i] = C * conv
    new_state = np.stack([hist_bits[w], hist_bits[w + 1]]).astype(np.uint16)
    return y, new_state


def shared_conv(table, X, W, states):
    """Conv over every row of a shared round.

    X: uint16 [R][6144]; W: uint16 [2048][3]; states: list (one per stream) of
    uint16 [2][2048]. Returns (y float64 [R][2048], list of new states).
    """
    X = np.asarray(X, dtype=np.uint16)
    R = table.n_rows
    y = np.zeros((R, HIDDEN), dtype=np.float64)
    new_states = []
    for s in range(len(table.rows)):
        r0, r1 = int(table.seg_off[s]), int(table.seg_off[s + 1])
        ys, st = replay_stream(X[r0:r1], W, states[s])
        y[r0:r1] = ys
        new_states.append(st)
    return y, new_states
