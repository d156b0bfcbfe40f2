"""Pins of the oracle's attention, partials and merge (CPU only).

Dense attention is pinned to torch's scaled_dot_product_attention in float64
(a library routine, with its own default scale 1/sqrt(64) and an explicit
boolean causal mask), to a hand-derived golden case, and to closed forms
(constant V, zero q, one visible key, GQA grouping). The partials are pinned
per split to the same library routine restricted to the split's keys and to
torch.logsumexp; the merge is pinned to dense attention (it must reproduce it
for every split size); causality and the per-stream independence of a shared
round are checked by perturbation.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attn, bf16, table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(vals):
    return bf16.round_f64(np.asarray(vals, dtype=np.float64))


def _round(streams, seed):
    rng = np.random.default_rng(seed)
    t = table.build(streams)
    Q = _bits(rng.standard_normal((t.n_rows, 32, 64)))
    K = [_bits(rng.standard_normal((8, cap, 64))) for (_, _, cap) in streams]
    V = [_bits(rng.standard_normal((8, cap, 64))) for (_, _, cap) in streams]
    return t, Q, K, V


def _sdpa_rows(t, Q, K, V, rows, lo=None, hi=None):
    """torch SDPA in float64 per row, keys [lo, hi) of what the row sees."""
    out = {}
    for r in rows:
        s = int(t.row_stream[r])
        n = int(t.row_nkeys[r])
        a = 0 if lo is None else lo
        b = n if hi is None else min(hi, n)
        q = torch.from_numpy(bf16.to_f64(Q[r])).reshape(1, 32, 1, 64)
        # slice to the visible keys (SDPA would multiply masked weights by
        # poisoned slots), then mask the ones before the split
        kk = torch.from_numpy(bf16.to_f64(K[s][:, :b])).repeat_interleave(4, dim=0)
        vv = torch.from_numpy(bf16.to_f64(V[s][:, :b])).repeat_interleave(4, dim=0)
        mask = torch.zeros(1, 1, 1, b, dtype=torch.bool)
        mask[..., a:b] = True
        o = F.scaled_dot_product_attention(q, kk[None], vv[None], attn_mask=mask)
        out[r] = o.reshape(32, 64).numpy()
    return out


def test_dense_matches_torch_sdpa():
    streams = [(1, 37, 64), (3, 100, 128), (5, 64, 64), (2, 2, 32)]
    t, Q, K, V = _round(streams, 1)
    # poison the slots past each stream's count: they must never be read
    for s, (_, k, cap) in enumerate(streams):
        K[s][:, k:] = 0x7FC0
        V[s][:, k:] = 0x7FC0
    ours = attn.attention(t, Q, K, V)
    ref = _sdpa_rows(t, Q, K, V, range(t.n_rows))
    for r in range(t.n_rows):
        assert np.allclose(ours[r], ref[r], rtol=0, atol=1e-12)


def test_golden_hand_case():
    with open(os.path.join(GOLDEN, "attn_hand.json")) as f:
        g = json.load(f)
    t = table.build([(1, 2, 32)])
    Q = np.zeros((1, 32, 64), dtype=np.uint16)
    Q[0, :, 0] = _bits(8.0)
    K = np.zeros((8, 32, 64), dtype=np.uint16)
    V = np.zeros((8, 32, 64), dtype=np.uint16)
    K[:, 1, 0] = _bits(1.0)
    V[:, 0, 0] = _bits(1.0)
    V[:, 1, 1] = _bits(1.0)
    o = attn.attention(t, Q, [K], [V])
    assert np.allclose(o[0, :, :2], np.array(g["o_first_two"])[None, :], rtol=0, atol=1e-15)
    assert np.all(o[0, :, 2:] == 0)
    po, pm, pl, d = attn.partials(t, Q, [K], [V])
    assert d.all()
    assert np.allclose(pm, g["m"]) and np.allclose(pl, g["l"], rtol=1e-15)
    assert np.allclose(po[:, :2], np.array(g["o_first_two"])[None, :], atol=1e-15)


def test_closed_forms():
    streams = [(4, 200, 224)]
    t, Q, K, V = _round(streams, 2)
    # V constant c in every slot -> o = c
    Vc = [np.full_like(V[0], _bits(0.75))]
    assert np.allclose(attn.attention(t, Q, K, Vc), 0.75, atol=1e-14)
    # q = 0 -> uniform weights -> mean of the visible V rows
    Q0 = np.zeros_like(Q)
    o = attn.attention(t, Q0, K, V)
    for r in range(t.n_rows):
        n = t.row_nkeys[r]
        for h in range(32):
            assert np.allclose(o[r, h], bf16.to_f64(V[0][h // 4, :n]).mean(axis=0), atol=1e-13)
    # one visible key -> V[0]
    t1 = table.build([(1, 1, 32)])
    o1 = attn.attention(t1, Q[:1], K, V)
    for h in range(32):
        assert np.array_equal(o1[0, h], bf16.to_f64(V[0][h // 4, 0]))
    # GQA: V of kv head g constant g -> q head h outputs floor(h/4)
    Vg = np.zeros_like(V[0])
    for g in range(8):
        Vg[g] = _bits(float(g))
    og = attn.attention(t, Q, K, [Vg])
    for h in range(32):
        assert np.allclose(og[:, h], h // 4, atol=1e-13)


def test_causality_keys_past_count_are_not_read():
    streams = [(6, 90, 96)]
    t, Q, K, V = _round(streams, 3)
    base = attn.attention(t, Q, K, V)
    for r in range(t.n_rows):
        n = t.row_nkeys[r]
        K2, V2 = K[0].copy(), V[0].copy()
        K2[:, n:] = _bits(50.0)
        V2[:, n:] = _bits(-7.0)
        o = attn.attention(t, Q, [K2], [V2], rows=[r])
        assert np.array_equal(o[r], base[r])


@pytest.mark.parametrize("streams", [
    [(1, 2500, 2560)],                 # 4 splits of 640
    [(3, 2500, 2560), (1, 513, 544)],  # 3 splits of 864, one of 513, ragged ends
    [(7, 4100, 4128)],                 # 3 splits of 1,376, the last 1,348 keys
    [(20, 9000, 9024)],                # two tiles, two split sizes: 5,024 then 3,976 keys
    [(16, 15000, 15008)],              # 5,376 x 2 then 4,248 keys
])
def test_partials_per_split_and_merge(streams):
    t, Q, K, V = _round(streams, 4)
    po, pm, pl, defined = attn.partials(t, Q, K, V)
    dense = attn.attention(t, Q, K, V)
    merged = attn.merge(t, po, pm, pl)
    assert np.allclose(merged, dense, rtol=0, atol=1e-12)
    for r in range(t.n_rows):
        s = int(t.row_stream[r])
        n = int(t.row_nkeys[r])
        for sp in range(int(t.nsplit[s])):
            recs = [t.record(r, h, sp) for h in range(32)]
            assert defined[recs].all()
            lo, hi = t.split_range(s, sp)
            hi = min(hi, n)
            if hi <= lo:
                assert np.all(pm[recs] == -np.inf) and np.all(pl[recs] == 0) and np.all(po[recs] == 0)
                continue
            if sp % 2 == 1 and r % 3 != 0:
                continue  # library cross-check on a subset keeps the test fast
            ref = _sdpa_rows(t, Q, K, V, [r], lo, hi)[r]
            assert np.allclose(po[recs], ref, atol=1e-12)
            q = torch.from_numpy(bf16.to_f64(Q[r])).reshape(32, 64)
            k = torch.from_numpy(bf16.to_f64(K[s][:, lo:hi])).repeat_interleave(4, dim=0)
            sc = torch.einsum("hd,hkd->hk", q, k) / math.sqrt(64)
            assert np.allclose(pm[recs], sc.max(dim=1).values.numpy(), atol=1e-12)
            lse = torch.logsumexp(sc, dim=1).numpy()
            assert np.allclose(pl[recs], np.exp(lse - pm[recs]), rtol=1e-12)


def test_shared_round_rows_equal_each_stream_alone():
    streams = [(2, 700, 704), (5, 300, 320), (1, 1500, 1536)]
    t, Q, K, V = _round(streams, 6)
    full = attn.attention(t, Q, K, V)
    for s, st_ in enumerate(streams):
        r0, r1 = t.seg_off[s], t.seg_off[s + 1]
        ta = table.build([st_])
        alone = attn.attention(ta, Q[r0:r1], [K[s]], [V[s]])
        assert np.array_equal(alone, full[r0:r1])


def test_merge_skips_empty_splits_and_propagates_nan():
    streams = [(1, 2500, 2560)]                      # 4 splits of 640
    t, Q, K, V = _round(streams, 8)
    po, pm, pl, _ = attn.partials(t, Q, K, V)
    base = attn.merge(t, po, pm, pl)
    # an empty split (m = -inf, l = 0, o = 0) changes nothing: drop split 1 of
    # head 0 from the reference by hand and compare with the merge of the rest
    recs = [t.record(0, 0, sp) for sp in range(4)]
    keep = [recs[0], recs[2], recs[3]]
    M = max(pm[x] for x in keep)
    wts = np.array([np.exp(pm[x] - M) * pl[x] for x in keep])
    by_hand = (wts[:, None] * po[keep]).sum(axis=0) / wts.sum()
    pm2, pl2, po2 = pm.copy(), pl.copy(), po.copy()
    pm2[recs[1]], pl2[recs[1]], po2[recs[1]] = -np.inf, 0.0, 0.0
    out = attn.merge(t, po2, pm2, pl2)
    assert np.allclose(out[0, 0], by_hand, atol=1e-14)
    assert np.array_equal(out[0, 1:], base[0, 1:])
    # a NaN partial is not an empty one: it reaches the output
    pl3 = pl.copy()
    pl3[recs[2]] = np.nan
    assert np.isnan(attn.merge(t, po, pm, pl3)[0, 0]).all()


# ------------------------------------------------------------ block attention
# PR #1391 "lfm2: draft with LiquidAI's DSpark drafter (--drafter)", its list
# of new kernels: the target's attention with a FULL flag, every block row
# seeing the keys [0, len + 1); read as every row seeing all K_s keys.

def test_block_matches_torch_sdpa_over_all_keys():
    streams = [(5, 200, 224), (1, 77, 96), (9, 600, 608)]
    t, Q, K, V = _round(streams, 11)
    tb = table.build(streams, full=True)
    assert all(int(tb.row_nkeys[r]) == streams[int(tb.row_stream[r])][1] for r in range(tb.n_rows))
    got = attn.attention(tb, Q, K, V)
    ref = _sdpa_rows(tb, Q, K, V, range(tb.n_rows))
    for r in range(tb.n_rows):
        assert np.allclose(got[r], ref[r], rtol=0, atol=1e-12), r


def test_block_last_row_and_one_row_windows_equal_causal():
    streams = [(4, 300, 320), (1, 90, 96), (16, 700, 704)]
    t, Q, K, V = _round(streams, 12)
    tb = table.build(streams, full=True)
    causal = attn.attention(t, Q, K, V)
    block = attn.attention(tb, Q, K, V)
    for s in range(len(streams)):
        last = int(t.seg_off[s + 1]) - 1          # the window's last row sees every key either way
        assert np.array_equal(block[last], causal[last])
    one = [(1, 50, 64), (1, 300, 320)]
    t1 = table.build(one)
    tb1 = table.build(one, full=True)
    assert np.array_equal(t1.row_nkeys, tb1.row_nkeys)
    assert np.array_equal(t1.work, tb1.work)


def test_block_rows_with_one_query_agree_and_causal_rows_do_not():
    streams = [(6, 400, 416)]
    t, Q, K, V = _round(streams, 13)
    Q[:] = Q[0]                                    # every row asks the same query
    tb = table.build(streams, full=True)
    block = attn.attention(tb, Q, K, V)
    causal = attn.attention(t, Q, K, V)
    for r in range(1, 6):
        assert np.array_equal(block[r], block[0])
        assert not np.array_equal(causal[r], causal[0])


def test_block_keys_past_count_unread_and_partials_merge():
    streams = [(20, 9000, 9024), (3, 2500, 2560)]
    t, Q, K, V = _round(streams, 14)
    tb = table.build(streams, full=True)
    base = attn.attention(tb, Q, K, V)
    K2 = [k.copy() for k in K]
    V2 = [v.copy() for v in V]
    for s, (_, n, _) in enumerate(streams):
        K2[s][:, n:] = _bits(50.0)
        V2[s][:, n:] = _bits(-7.0)
    assert np.array_equal(attn.attention(tb, Q, K2, V2), base)
    po, pm, pl, defined = attn.partials(tb, Q, K, V)
    assert defined.all()                           # every row has every split of its stream
    assert np.allclose(attn.merge(tb, po, pm, pl), base, rtol=0, atol=1e-12)
