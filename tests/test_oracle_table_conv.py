"""Pins of the oracle's segment table and conv replay (CPU only).

Table: the hand-derived golden table of the tiny workload, invariants that
hold for any valid round (rows partition [0, R); tiles stay inside a stream
with at most 16 rows; visible counts run up to K_s; partial records of
distinct (row, head, split) are distinct and fill [0, partial_count)), brute
force over random small rounds, and the partial counts at 1, 32 and 2,048
rows (the sizes the pages' table test names).

Conv: a hand-derived golden window, closed forms for one-hot taps, the
channel-wise numpy.correlate of the history (a library routine), and the
invariant that a window equals one-row calls carried through the state.
"""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import bf16, conv, table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ table

def test_table_golden_tiny():
    with open(os.path.join(GOLDEN, "table_tiny.json")) as f:
        g = json.load(f)
    t = table.build([tuple(s) for s in g["streams"]])
    assert t.seg_off.tolist() == g["seg_off"]
    assert t.row_stream.tolist() == g["row_stream"]
    assert t.row_pos.tolist() == g["row_pos"]
    assert t.row_nkeys.tolist() == g["row_nkeys"]
    assert t.split.tolist() == g["split"]
    assert t.nsplit.tolist() == g["nsplit"]
    assert t.poff.tolist() == g["poff"]
    assert t.partial_count == g["partial_count"]
    assert t.tiles.tolist() == g["tiles"]
    assert len(t.work) == g["n_work"]


def _check_invariants(streams, t):
    S = len(streams)
    R = sum(w for w, _, _ in streams)
    assert t.n_rows == R
    # rows partition [0, R) in caller order
    seen = np.zeros(R, dtype=int)
    for s in range(S):
        seen[t.seg_off[s]:t.seg_off[s + 1]] += 1
        assert t.seg_off[s + 1] - t.seg_off[s] == streams[s][0]
    assert (seen == 1).all()
    for r in range(R):
        s = t.row_stream[r]
        w, k, _ = streams[s]
        assert t.seg_off[s] <= r < t.seg_off[s + 1]
        assert 1 <= t.row_nkeys[r] <= k
        if t.row_pos[r] == w - 1:
            assert t.row_nkeys[r] == k
    # tiles: inside a stream, <= 16 rows, cover every row once
    cover = np.zeros(R, dtype=int)
    for (s, r0, n, p0) in t.tiles:
        assert 1 <= n <= 16
        assert t.seg_off[s] + p0 == r0 and p0 + n <= streams[s][0]
        cover[r0:r0 + n] += 1
    assert (cover == 1).all()
    # records: a bijection from (row, head, split < nsplit_s) onto [0, P)
    recs = []
    for r in range(R):
        s = t.row_stream[r]
        for h in range(32):
            for sp in range(t.nsplit[s]):
                recs.append(t.record(r, h, sp))
    assert sorted(recs) == list(range(t.partial_count))
    # each stream's records form one contiguous range of its own
    for s in range(S):
        lo = t.poff[s]
        hi = lo + t.nsplit[s] * streams[s][0] * 32
        mine = [t.record(r, h, sp) for r in range(t.seg_off[s], t.seg_off[s + 1])
                for h in range(32) for sp in range(t.nsplit[s])]
        assert min(mine) == lo and max(mine) == hi - 1
    # work: a one-tile stream's tile, a longer stream's groups of 4 tiles,
    # each with every (kv head, split) holding a key its last row sees
    want = set()
    for s in range(S):
        mine = [ti for ti, tt in enumerate(t.tiles) if tt[0] == s]
        size = len(mine) if len(mine) == 1 else 4
        for i in range(0, len(mine), size):
            grp = mine[i:i + size]
            _s, _r0, n, p0 = t.tiles[grp[-1]]
            last = streams[s][1] - streams[s][0] + p0 + n
            for sp in range(t.nsplit[s]):
                if t.bounds[s][sp] < last:
                    for g in range(8):
                        want.add((grp[0], g, sp, len(grp)))
    got = [tuple(x) for x in t.work.tolist()]
    assert len(got) == len(set(got)) and set(got) == want
    # every tile of every stream is in exactly one group, groups of 1 only
    # for one-tile streams
    firsts = {}
    for ti, _g, _sp, n in got:
        firsts[ti] = n
    covered = sorted(ti + k for ti, n in firsts.items() for k in range(n))
    assert covered == list(range(len(t.tiles)))
    for ti, n in firsts.items():
        s = t.tiles[ti][0]
        assert all(t.tiles[ti + k][0] == s for k in range(n))
        assert (n == 1) == (sum(1 for tt in t.tiles if tt[0] == s) == 1)


_stream = st.integers(1, 40).flatmap(
    lambda w: st.integers(w, 9000).map(lambda k: (w, k, ((k + 31) // 32) * 32)))


@settings(max_examples=60, deadline=None)
@given(st.lists(_stream, min_size=1, max_size=6))
def test_table_invariants_random(streams):
    _check_invariants(streams, table.build(streams))


def test_table_split_plan_by_window():
    # the cap depends only on the stream's own rows
    assert [table.split_cap(w) for w in (1, 2, 3, 4, 5, 8, 9, 16, 17, 512)] == \
        [768, 768, 1024, 1024, 2560, 2560, 7168, 7168, 5120, 5120]
    # windows of up to 8 rows, equal splits by hand: 1,000 / 2 = 500 -> 512;
    # 100 / 1 -> 128; 4,096 / ceil(4,096 / 768) = 4,096 / 6 = 682.7 -> 704;
    # 32,768 / ceil(32,768 / 2,560) = 32,768 / 13 = 2,520.6 -> 2,528 (cap 2,560)
    assert [table.split_plan(w, k) for (w, k) in ((1, 1000), (3, 100), (1, 4096), (8, 32768))] == \
        [(512, 512, 2, 2), (128, 128, 1, 1), (704, 704, 6, 6), (2528, 2528, 13, 13)]
    # 16-row tiles, two sizes by hand (A = ceil(5K / (5b + 4(n - b))) up to 32,
    # B = ceil((K - bA) / (n - b)) up to 32):
    #   65,536: n = 10, b = 5: A = ceil(327,680 / 45) = 7,282 -> 7,296,
    #           B = ceil(29,056 / 5) = 5,812 -> 5,824; last split [59,776, 65,536)
    #   98,304: n = 14, b = 7: A = ceil(491,520 / 63) = 7,802 -> 7,808,
    #           B = ceil(43,648 / 7) = 6,236 -> 6,240; last split [92,096, 98,304)
    #  131,072: n = 19, b = 10: A = ceil(655,360 / 86) = 7,621 -> 7,648,
    #           B = ceil(54,592 / 9) = 6,066 -> 6,080; last split [125,120, 131,072)
    #    7,169: n = 2, b = 1: A = ceil(35,845 / 9) = 3,983 -> 4,000, B = 3,169 -> 3,200
    #    7,000: n = 1: one split of 7,008
    assert [table.split_plan(16, k) for k in (65536, 98304, 131072, 7169, 7000)] == \
        [(7296, 5824, 5, 10), (7808, 6240, 7, 14), (7648, 6080, 10, 19), (4000, 3200, 1, 2),
         (7008, 7008, 1, 1)]
    assert table.split_bounds(16, 65536).tolist() == \
        [0, 7296, 14592, 21888, 29184, 36480, 42304, 48128, 53952, 59776, 65536]
    # prompt chunks (more than 16 rows) take the 5,120 cap, two sizes by hand:
    #  131,072: n = 26, b = 13: A = ceil(655,360 / 117) = 5,602 -> 5,632,
    #           B = ceil(57,856 / 13) = 4,451 -> 4,480; last split [126,976, 131,072)
    assert table.split_plan(17, 131072) == (5632, 4480, 13, 26)
    assert table.split_bounds(17, 131072)[-2:].tolist() == [126976, 131072]


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 16), st.integers(1, 131072))
def test_table_split_plan_properties(rows, keys):
    cap = table.split_cap(rows)
    A, B, b, n = table.split_plan(rows, keys)
    bounds = table.split_bounds(rows, keys)
    sizes = np.diff(bounds)
    assert n == -(-keys // cap)                  # as many splits as the cap forces
    assert len(sizes) == n and bounds[0] == 0 and bounds[-1] == keys
    assert (sizes > 0).all() and (bounds[:-1] % 32 == 0).all()
    if min(rows, 16) <= 8 or n == 1:             # equal splits, every one but the last full
        assert A == B and b == n and A % 32 == 0 and A <= cap
        assert (sizes[:-1] == A).all() and 0 < sizes[-1] <= A
    else:                                        # the first half 5/4 the size of the rest
        assert b == -(-n // 2) and A % 32 == 0 and B % 32 == 0
        assert (sizes[:b] == A).all() and (sizes[b:-1] == B).all() and 0 < sizes[-1] <= B
        assert 1.1 < A / B < 1.45 and A <= cap * 5 // 4 + 32


@pytest.mark.parametrize("rows,expect", [
    # 1 row, 1 stream of 4096 keys: 6 splits of 704 -> 6 * 32 records
    ([(1, 4096, 4096)], 192),
    # 32 rows as 32 one-row streams of 1,000 keys: 2 splits each -> 32 * 2 * 32
    ([(1, 1000, 1024)] * 32, 2048),
    # 2,048 rows as 128 streams of 16 rows and 131,072 keys: 19 splits each
    ([(16, 131072, 131072)] * 128, 128 * 16 * 32 * 19),
])
def test_table_partial_counts_at_1_32_2048_rows(rows, expect):
    t = table.build(rows)
    assert t.n_rows in (1, 32, 2048)
    assert t.partial_count == expect


@pytest.mark.parametrize("bad", [
    [], [(0, 16, 32)], [(4, 3, 32)], [(1, 131073, 131104)], [(1, 64, 32)],
    [(1, 16, 48)], [(16, 32, 32)] * 129,
])
def test_table_refusals(bad):
    with pytest.raises(ValueError):
        table.build(bad)


# ------------------------------------------------------------------- conv

def _bits(vals):
    return bf16.round_f64(np.asarray(vals, dtype=np.float64))


def test_conv_golden_hand_window():
    with open(os.path.join(GOLDEN, "conv_hand.json")) as f:
        g = json.load(f)
    w = len(g["rows"])
    X = np.zeros((w, 6144), dtype=np.uint16)
    for i, row in enumerate(g["rows"]):
        X[i, 0], X[i, 2048], X[i, 4096] = _bits([row["B"], row["C"], row["x"]])
    W = np.zeros((2048, 3), dtype=np.uint16)
    W[0] = _bits(g["W"])
    st0 = np.zeros((2, 2048), dtype=np.uint16)
    st0[:, 0] = _bits(g["state"])
    y, new = conv.replay_stream(X, W, st0)
    assert y[:, 0].tolist() == g["y"]
    assert np.all(y[:, 1:] == 0)
    assert bf16.to_f64(new[:, 0]).tolist() == g["new_state"]
    rc = g["rounding_case"]
    X2 = np.zeros((1, 6144), dtype=np.uint16)
    X2[0, 0], X2[0, 4096] = int(rc["B_bits"], 16), int(rc["x_bits"], 16)
    _, new2 = conv.replay_stream(X2, W, st0)
    assert new2[1, 0] == int(rc["bx_bits"], 16)


def _rand_stream(rng, w):
    X = _bits(rng.standard_normal((w, 6144)))
    W = _bits(rng.standard_normal((2048, 3)) / np.sqrt(3))
    state = _bits(rng.standard_normal((2, 2048)))
    return X, W, state


def test_conv_one_hot_taps_closed_forms():
    rng = np.random.default_rng(5)
    X, _, state = _rand_stream(rng, 4)
    B, C, x = (bf16.to_f64(X[:, i * 2048:(i + 1) * 2048]) for i in range(3))
    bx = bf16.to_f64(bf16.round_f64(B * x))
    one = _bits(1.0)
    for k, expect in [
        (2, C * bx),                                                        # newest tap only
        (0, C * np.concatenate([bf16.to_f64(state), bx[:2]])),              # oldest tap only
        (1, C * np.concatenate([bf16.to_f64(state[1:]), bx[:3]])),          # middle tap only
    ]:
        W = np.zeros((2048, 3), dtype=np.uint16)
        W[:, k] = one
        y, _ = conv.replay_stream(X, W, state)
        assert np.array_equal(y, expect)


def test_conv_matches_numpy_correlate_per_channel():
    rng = np.random.default_rng(9)
    w = 6
    X, W, state = _rand_stream(rng, w)
    y, new = conv.replay_stream(X, W, state)
    B, C, x = (bf16.to_f64(X[:, i * 2048:(i + 1) * 2048]) for i in range(3))
    bx = bf16.to_f64(bf16.round_f64(B * x))
    hist = np.concatenate([bf16.to_f64(state), bx])          # [w+2][2048]
    Wf = bf16.to_f64(W)
    for c in range(0, 2048, 97):
        ref = C[:, c] * np.correlate(hist[:, c], Wf[c], mode="valid")
        assert np.allclose(y[:, c], ref, rtol=1e-14, atol=1e-14)
    assert np.array_equal(bf16.to_f64(new), hist[-2:])


@pytest.mark.parametrize("w", [1, 2, 3, 7])
def test_conv_window_equals_one_row_calls(w):
    rng = np.random.default_rng(100 + w)
    X, W, state = _rand_stream(rng, w)
    y, new = conv.replay_stream(X, W, state)
    st_ = state.copy()
    for i in range(w):
        yi, st_ = conv.replay_stream(X[i:i + 1], W, st_)
        assert np.array_equal(yi[0], y[i])
    assert np.array_equal(st_, new)


def test_conv_shared_round_is_per_stream():
    rng = np.random.default_rng(21)
    streams = [(1, 16, 32), (3, 40, 64), (2, 8, 32)]
    t = table.build(streams)
    X = _bits(rng.standard_normal((t.n_rows, 6144)))
    W = _bits(rng.standard_normal((2048, 3)))
    states = [_bits(rng.standard_normal((2, 2048))) for _ in streams]
    y, new = conv.shared_conv(t, X, W, states)
    for s in range(3):
        r0, r1 = t.seg_off[s], t.seg_off[s + 1]
        ys, ns = conv.replay_stream(X[r0:r1], W, states[s])
        assert np.array_equal(y[r0:r1], ys) and np.array_equal(new[s], ns)
