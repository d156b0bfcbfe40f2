"""float64 GQA attention, split-K partials and their merge (oracle; test only).

PR #1377 "LFM2: shared-round decode", shared-round commit: one attention
launch a layer over every stream's rows, each stream's partials kept apart in
the scratch, and the stream attention checked against float64 attention; the
inline-bodies commit names the per-row attention and merge bodies. Issue
#1374 "LFM2.5-24B-A2B on Metal ..." (Design, and the DSpark PR #1391's
drafter notes) contrasts the target's causal count with a FULL block that
sees every key. The pages print no formula; the readings here are:

* GQA with 32 q heads over 8 kv heads, head dim 64; q head h reads kv head
  floor(h / 4);
* score s_j = 0.125 * (q . k_j), 0.125 = 1/sqrt(64);
* row r sees keys j < n_r (the table's causal count), softmax over them,
  output o = sum_j softmax(s)_j v_j;
* split t of stream s covers its keys of the split plan (oracle.table)
  intersected with the row's visible keys and gives (m_t, l_t, o_t): the
  max score, the sum of
  exp(s_j - m_t), and the exp-weighted mean of v_j; an empty split gives
  (-inf, 0, 0);
* the merge takes M = max_t m_t and returns
  sum_t exp(m_t - M) l_t o_t / sum_t exp(m_t - M) l_t over the row's splits
  in split order, skipping empty ones (l = 0); a NaN in any partial makes
  the output NaN.

K and V are given per stream in their logical layout [8][keys][64] (bf16 bit
patterns); only the first K_s keys are read.
"""

import numpy as np

from . import bf16
from .table import N_KV_HEADS, N_Q_HEADS

HEAD_DIM = 64
GROUP = N_Q_HEADS // N_KV_HEADS
SCALE = 0.125


def _scores(q, k):
    """q: float64 [n_q][64]; k: float64 [n][64] -> 0.125 * q k^T."""
    return SCALE * (q @ k.T)


def attention(table, Q, K_list, V_list, rows=None):
    """Dense causal softmax attention, float64. Returns o [R][32][64].

    Only the listed rows (default: all) are computed; the others stay zero.
    """
    Q = np.asarray(Q, dtype=np.uint16)
    R = table.n_rows
    out = np.zeros((R, N_Q_HEADS, HEAD_DIM), dtype=np.float64)
    for r in (range(R) if rows is None else rows):
        s = int(table.row_stream[r])
        n = int(table.row_nkeys[r])
        for g in range(N_KV_HEADS):
            k = bf16.to_f64(K_list[s][g, :n])
            v = bf16.to_f64(V_list[s][g, :n])
            q = bf16.to_f64(Q[r, g * GROUP:(g + 1) * GROUP])
            sc = _scores(q, k)                       # [4][n]
            sc = sc - sc.max(axis=1, keepdims=True)
            p = np.exp(sc)
            out[r, g * GROUP:(g + 1) * GROUP] = (p @ v) / p.sum(axis=1, keepdims=True)
    return out


def partials(table, Q, K_list, V_list, rows=None):
    """Split-K partials for every record of the listed rows (default: all).

    Returns (o [P][64], m [P], l [P], defined [P] bool) over the table's
    partial_count records; ``defined`` marks the records of
    (row, head, split) with split < nsplit_s. Records of rows not listed stay
    undefined.
    """
    Q = np.asarray(Q, dtype=np.uint16)
    P = table.partial_count
    o = np.zeros((P, HEAD_DIM), dtype=np.float64)
    m = np.full(P, -np.inf, dtype=np.float64)
    l = np.zeros(P, dtype=np.float64)
    defined = np.zeros(P, dtype=bool)
    rows = range(table.n_rows) if rows is None else rows
    for r in rows:
        s = int(table.row_stream[r])
        n = int(table.row_nkeys[r])
        for g in range(N_KV_HEADS):
            q = bf16.to_f64(Q[r, g * GROUP:(g + 1) * GROUP])
            for t in range(int(table.nsplit[s])):
                lo, hi = table.split_range(s, t)
                hi = min(hi, n)
                for hh in range(GROUP):
                    rec = table.record(r, g * GROUP + hh, t)
                    defined[rec] = True
                if hi <= lo:
                    continue                          # empty: (-inf, 0, 0)
                k = bf16.to_f64(K_list[s][g, lo:hi])
                v = bf16.to_f64(V_list[s][g, lo:hi])
                sc = _scores(q, k)                    # [4][hi-lo]
                mt = sc.max(axis=1)
                p = np.exp(sc - mt[:, None])
                lt = p.sum(axis=1)
                ot = (p @ v) / lt[:, None]
                for hh in range(GROUP):
                    rec = table.record(r, g * GROUP + hh, t)
                    m[rec], l[rec], o[rec] = mt[hh], lt[hh], ot[hh]
    return o, m, l, defined


def merge(table, o, m, l, rows=None):
    """Merge each row's partials in split order. Returns out [R][32][64]."""
    out = np.zeros((table.n_rows, N_Q_HEADS, HEAD_DIM), dtype=np.float64)
    rows = range(table.n_rows) if rows is None else rows
    for r in rows:
        nt = table.row_nsplit(r)
        for h in range(N_Q_HEADS):
            recs = [table.record(r, h, t) for t in range(nt)]
            recs = [x for x in recs if l[x] != 0.0]      # empty splits only
            if not recs:
                continue
            M = np.max(m[recs])                          # NaN propagates
            num = np.zeros(HEAD_DIM, dtype=np.float64)
            den = 0.0
            for x in recs:
                wgt = np.exp(m[x] - M) * l[x]
                num += wgt * o[x]
                den += wgt
            out[r, h] = num / den
    return out
