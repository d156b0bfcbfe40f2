"""Markov-head step of the drafter: score, pick and flag of every drafted row
(oracle; test infrastructure only).

PR #1391 "lfm2: draft with LiquidAI's DSpark drafter (--drafter)", its
description and list of new kernels: the drafter's Markov head scores each
row of the block as its logits plus W2 . W1[token before the row] and takes
that row's argmax before the next row, which uses the pick as its previous
token; the step kernels gather W1's row, take the W2 dot (bf16 weights by
default: the bf16 scan), add it to the row's logits and pick the argmax,
ties to the lowest token, a NaN score flagged. The PR's testing notes give
the family test's rule, the argmax of bf16(base + bf16(W2 . W1[prev])), and
the step's contract shape 1 x 128,000 x 256 (rows x vocabulary x rank); the
review's config admission caps the rank at 256 (W1's row is staged in 256
floats) and its 4-bit finding gives W2 as 128,000 x 256 (vocabulary x rank).

Readings taken where the pages leave a step open (listed in the design notes):

* dot_v = sum over k of W2[v][k] * W1[prev][k], accumulated in float32
  with k ascending from 0 and one rounding per term (the product of two
  bf16 values is exact in float32, so a fused multiply-add and a multiply
  then add agree); the pages fix float32 for neither the dot nor its order,
  this is the plainest float32 dot;
* score_v = bf16(fl32(base_v + bf16(dot_v))), each bf16() round to nearest,
  ties to even;
* pick and flag follow the greedy pick of the target's rows: the first
  largest score, NaN skipped, -0 equal to +0, a row without a non-NaN score
  picks 0; the flag is set by a NaN or an infinity among the scores (the
  pick's nonfinite flag, which the held-draft fix carries to the verify);
* a chain is (row0, depth): rows row0 .. row0 + depth - 1 of the block, one
  row after the other; the first row's previous token is given (the pending
  token), row j's is the pick of row j - 1;
* a previous token outside [0, vocab) flags its row and adds nothing (the
  dot is taken as +0), so nothing is read outside W1.

Weights and logits are uint16 bf16 bit patterns. ``dot`` is the float32
accumulation written out over k; everything else is float64 arithmetic
rounded where the readings say. Adding two float32-representable values in
float64 and rounding the result to float32 gives the correctly rounded
float32 sum (float64 carries more than 2 x 24 + 2 bits), so each float32
rounding here is a single rounding of the exact value. The float32 rounding
of base + bf16(dot) is kept as the rule writes it, though it cannot change
the score: the sum of two bf16 values is exact in float32 unless their
exponents lie so far apart that the sum sits far from every bf16 midpoint,
so rounding it through float32 to bf16 equals rounding it once.
"""

import numpy as np

from . import argmax as _argmax
from . import bf16


def dot(w2, e):
    """float32 dot of every row of W2 with one W1 row.

    w2: uint16 [V][R] bf16 bits; e: uint16 [R] bf16 bits. Returns float32 [V]:
    acc = 0; for k = 0 .. R-1: acc = fl32(acc + W2[v][k] * e[k])."""
    W = bf16.to_f64(np.asarray(w2, dtype=np.uint16))
    E = bf16.to_f64(np.asarray(e, dtype=np.uint16))
    acc = np.zeros(W.shape[0], dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        for k in range(W.shape[1]):
            acc = (acc.astype(np.float64) + W[:, k] * E[k]).astype(np.float32)
    return acc


def scores(base_row, w1, w2, prev):
    """Scores of one row: uint16 [V] bf16 bits, and whether prev was valid."""
    base = bf16.to_f64(np.asarray(base_row, dtype=np.uint16))
    V = base.shape[0]
    valid = 0 <= int(prev) < V
    if valid:
        d = bf16.to_f64(bf16.round_f64(dot(w2, np.asarray(w1)[int(prev)]).astype(np.float64)))
    else:
        d = np.zeros(V)
    with np.errstate(invalid="ignore", over="ignore"):
        t = (base + d).astype(np.float32).astype(np.float64)
    return bf16.round_f64(t), valid


def markov_pick(base, chains, prev0, w1, w2, pick, flag):
    """Run every chain. base: uint16 [rows][V] (the block rows' logits);
    chains: [(row0, depth)]; prev0: the first previous token of each chain;
    w1, w2: uint16 [V][R]. pick (int32 [rows]) and flag (uint8 [rows]) are
    written at the chains' rows only."""
    base = np.asarray(base, dtype=np.uint16)
    for (row0, depth), p0 in zip(chains, prev0):
        prev = int(p0)
        for j in range(max(0, int(depth))):
            r = int(row0) + j
            s, valid = scores(base[r], w1, w2, prev)
            pk, fl = _argmax.row_argmax(s[None, :])
            pick[r] = pk[0]
            flag[r] = np.uint8(1 if (fl[0] or not valid) else 0)
            prev = int(pk[0])
    return pick, flag
