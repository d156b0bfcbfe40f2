"""Pins of the Markov-step oracle (PR #1391, description: each drafted row
is scored as its logits plus W2 . W1[token before the row], rows taken in
order with each pick feeding the next row; lowest token on a tie; a NaN
score flagged; the testing notes' rule bf16(base + bf16(W2 . W1[prev]))).

Pinned against: a hand-derived accumulation-order fixture, integer weights
(the dot exact in any order) with torch's own bf16 rounding for the two
roundings, permutation chains (a transposed W2, a column gather of W1 or a
wrong previous token each pick other tokens), the greedy-pick special cases,
and the float32 summation error bound against math.fsum."""

import json
import math
import os

import numpy as np
import torch

from oracle import markov

HERE = os.path.dirname(__file__)
QNAN, POS_INF, NEG_INF, NEG_ZERO = 0x7FC0, 0x7F80, 0xFF80, 0x8000


def bits(x):
    """float values exactly representable in bf16 -> uint16 bit patterns."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def rand_bf16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape).astype(np.float32) * np.float32(scale)).view(np.uint32).__rshift__(16).astype(np.uint16)


def torch_bf16_bits(t32):
    return t32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_accumulation_order_golden():
    g = json.load(open(os.path.join(HERE, "golden", "markov_order.json")))
    w2 = bits(np.array([g["w2_row"]], dtype=np.float32))
    for case in g["cases"]:
        got = markov.dot(w2, bits(np.array(case["e"], dtype=np.float32)))
        assert got.dtype == np.float32
        assert float(got[0]) == case["dot"], case["derivation"]


def test_integer_weights_dot_is_exact():
    rng = np.random.default_rng(1)
    V, R = 300, 256
    W = rng.integers(-8, 9, (V, R))
    e = rng.integers(-8, 9, R)
    got = markov.dot(bits(W.astype(np.float32)), bits(e.astype(np.float32)))
    assert np.array_equal(got.astype(np.int64), W @ e)


def test_integer_weights_scores_against_torch_rounding():
    """dot exact (|dot| <= 256 * 64 < 2^24); the two bf16 roundings and the
    float32 add are torch's. Dots past 256 are not all bf16 values, so the
    inner rounding matters; the test checks that it does."""
    rng = np.random.default_rng(2)
    V, R = 2000, 256
    W1 = rng.integers(-8, 9, (V, R))
    W2 = rng.integers(-8, 9, (V, R))
    base = rand_bf16(rng, V, scale=300.0)
    prev = 17
    s, valid = markov.scores(base, bits(W1.astype(np.float32)), bits(W2.astype(np.float32)), prev)
    assert valid
    exact = torch.tensor((W2 @ W1[prev]).astype(np.float32))
    d = exact.to(torch.bfloat16).float()
    b = torch.from_numpy(base.view(np.int16)).view(torch.bfloat16).float()
    want = torch_bf16_bits(b + d)
    assert np.array_equal(s, want)
    without_inner = torch_bf16_bits(b + exact)
    assert not np.array_equal(without_inner, want)


def _perm_weights(V, sigma, tau):
    """W1[p] = one-hot(tau[p]); W2[v][k] = 4 where v = sigma[k]: the dot of
    row v with W1[p] is 4 when v = sigma[tau[p]], else 0."""
    W1 = np.zeros((V, V), dtype=np.float32)
    W1[np.arange(V), tau] = 1.0
    W2 = np.zeros((V, V), dtype=np.float32)
    W2[sigma, np.arange(V)] = 4.0
    return bits(W1), bits(W2)


def test_chains_follow_the_previous_pick():
    V = 16
    sigma = (5 * np.arange(V) + 3) % V
    tau = (3 * np.arange(V) + 7) % V
    W1, W2 = _perm_weights(V, sigma, tau)
    base = np.zeros((8, V), dtype=np.uint16)
    pick = np.full(8, -1, dtype=np.int32)
    flag = np.full(8, 9, dtype=np.uint8)
    markov.markov_pick(base, [(0, 5), (6, 2)], [3, 11], W1, W2, pick, flag)
    want, p = [], 3
    for _ in range(5):
        p = int(sigma[tau[p]])
        want.append(p)
    p = 11
    want2 = []
    for _ in range(2):
        p = int(sigma[tau[p]])
        want2.append(p)
    assert pick[:5].tolist() == want and pick[6:8].tolist() == want2
    assert pick[5] == -1 and flag[5] == 9           # not in a chain: untouched
    assert flag[[0, 1, 2, 3, 4, 6, 7]].tolist() == [0] * 7
    # planted mistakes give other picks: a transposed W2, W1's column
    for w1, w2 in ((W1, np.ascontiguousarray(W2.T)), (np.ascontiguousarray(W1.T), W2)):
        pk = np.zeros(8, dtype=np.int32)
        markov.markov_pick(base, [(0, 5)], [3], w1, w2, pk, np.zeros(8, dtype=np.uint8))
        assert pk[:5].tolist() != want


def test_chains_are_independent():
    rng = np.random.default_rng(4)
    V, R = 500, 32
    W1, W2 = rand_bf16(rng, (V, R)), rand_bf16(rng, (V, R))
    base = rand_bf16(rng, (7, V))
    both_p, both_f = np.zeros(7, np.int32), np.zeros(7, np.uint8)
    markov.markov_pick(base, [(0, 3), (3, 4)], [10, 20], W1, W2, both_p, both_f)
    a_p, a_f = np.zeros(7, np.int32), np.zeros(7, np.uint8)
    markov.markov_pick(base, [(3, 4)], [20], W1, W2, a_p, a_f)
    assert np.array_equal(both_p[3:], a_p[3:]) and np.array_equal(both_f[3:], a_f[3:])


def _one(base_vals, prev=0, V=None):
    base = bits(np.array(base_vals, dtype=np.float32)) if not isinstance(base_vals, np.ndarray) else base_vals
    V = len(base)
    W = np.zeros((V, 8), dtype=np.uint16)            # dot = +0 everywhere
    pick, flag = np.zeros(1, np.int32), np.zeros(1, np.uint8)
    markov.markov_pick(base[None, :], [(0, 1)], [prev], W, W, pick, flag)
    return int(pick[0]), int(flag[0])


def test_greedy_rule_special_cases():
    assert _one([1.0, 3.0, 3.0, 2.0]) == (1, 0)                  # tie: lowest token
    nan_row = bits(np.array([1.0, 5.0, 2.0, 0.0], dtype=np.float32))
    nan_row[1] = QNAN
    assert _one(nan_row) == (2, 1)                               # NaN skipped, flagged
    inf_row = bits(np.array([1.0, 5.0, 2.0, 0.0], dtype=np.float32))
    inf_row[3] = POS_INF
    assert _one(inf_row) == (3, 1)
    ninf = np.array([NEG_INF, NEG_INF, NEG_INF], dtype=np.uint16)
    assert _one(ninf) == (0, 1)
    assert _one(np.array([QNAN, QNAN], dtype=np.uint16)) == (0, 1)  # no real score: 0
    z = np.array([bits(np.float32(-1.0)), NEG_ZERO, 0x0000], dtype=np.uint16)
    assert _one(z) == (1, 0)                                     # -0 == +0 (+0 + -0 is +0)


def test_invalid_previous_token_flags_and_adds_nothing():
    rng = np.random.default_rng(5)
    V, R = 64, 16
    W1, W2 = rand_bf16(rng, (V, R)), rand_bf16(rng, (V, R))
    base = rand_bf16(rng, (3, V))
    for bad in (-1, V, 1 << 30):
        pick, flag = np.zeros(3, np.int32), np.zeros(3, np.uint8)
        markov.markov_pick(base, [(0, 3)], [bad], W1, W2, pick, flag)
        row = (base[0].astype(np.uint32) << 16).view(np.float32)
        assert flag[0] == 1 and pick[0] == int(np.argmax(row))   # the scores are the logits
        # the next row starts from that pick, valid again
        p1, f1 = np.zeros(3, np.int32), np.zeros(3, np.uint8)
        markov.markov_pick(base, [(1, 2)], [int(pick[0])], W1, W2, p1, f1)
        assert pick[1:].tolist() == p1[1:].tolist() and flag[1:].tolist() == f1[1:].tolist()


def test_float32_error_bound_against_fsum():
    rng = np.random.default_rng(6)
    V, R = 400, 256
    W2, e = rand_bf16(rng, (V, R)), rand_bf16(rng, R)
    got = markov.dot(W2, e)
    Wf = (W2.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ef = (e.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    u = 2.0 ** -24
    gamma = R * u / (1 - R * u)
    for v in range(V):
        terms = Wf[v] * ef
        exact = math.fsum(terms.tolist())
        assert abs(float(got[v]) - exact) <= gamma * math.fsum(np.abs(terms).tolist())
