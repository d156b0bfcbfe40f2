"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host table builder is bit-exact against the oracle's independent builder
(no GPU call is made here)."""

import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import workloads
from oracle import table as otable

asv = pytest.importorskip("attention_stream_verify_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    inc = os.path.join(ROOT, "include")
    src = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    return sorted(set(re.findall(r"\b(asv_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_what_the_binding_knows():
    assert _declared() == sorted(asv.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(asv._lib.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name
    assert asv.abi_version() == 4
    assert asv.strerror(-4) == "caller buffer too small"


def _fake_ptrs(streams, n_layers, nbytes_fn, base):
    """Distinct, 16-byte aligned, non-overlapping fake addresses (never dereferenced)."""
    out, addr = [], base
    for _ in range(n_layers):
        layer = []
        for s in streams:
            layer.append(addr)
            addr += ((nbytes_fn(s) + 4095) // 4096) * 4096
        out.append(layer)
    return out


def _build(streams, n_conv=1, n_attn=1, full=False):
    cs = _fake_ptrs(streams, n_conv, lambda s: 8192, 1 << 40)
    kp = _fake_ptrs(streams, n_attn, lambda s: 8 * s[2] * 64 * 2, 1 << 42)
    vp = _fake_ptrs(streams, n_attn, lambda s: 8 * s[2] * 64 * 2, 1 << 44)
    info, blob = asv.seg_table_build(streams, cs, kp, vp, full=full)
    return info, blob, asv.table_arrays(info, blob), (cs, kp, vp)


def _compare(streams, full=False):
    info, blob, t, (cs, kp, vp) = _build(streams, full=full)
    o = otable.build(streams, full=full)
    S, R = len(streams), o.n_rows
    assert (info.n_streams, info.n_rows, info.n_tiles) == (S, R, len(o.tiles))
    assert info.partial_count == o.partial_count
    segs = t["segs"]
    assert np.array_equal(segs["row0"], o.seg_off[:-1])
    assert np.array_equal(segs["rows"], o.rows) and np.array_equal(segs["keys"], o.keys)
    assert np.array_equal(segs["cap"], o.caps)
    assert np.array_equal(segs["split_keys"], o.split)
    assert np.array_equal(segs["nsplit"], o.nsplit)
    assert np.array_equal(segs["split_tail"], o.split_tail)
    assert np.array_equal(segs["nbig"], o.nbig)
    assert not segs["reserved"].any()
    assert np.array_equal(segs["poff"], o.poff)
    rows = t["rows"]
    assert np.array_equal(rows["stream"], o.row_stream)
    assert np.array_equal(rows["pos"], o.row_pos)
    assert np.array_equal(rows["nkeys"], o.row_nkeys)
    tiles = np.stack([t["tiles"][f] for f in ("stream", "row0", "nrows", "pos0")], axis=1)
    assert np.array_equal(tiles, o.tiles)
    for r in range(R):
        tt = o.tiles[rows["tile"][r]]
        assert tt[1] <= r < tt[1] + tt[2]
    # work items: the same set (their order is a schedule), keys = visited
    # keys, costliest first (a group's waves each walk every key)
    w = t["work"]
    got = sorted(zip(w["tile"].tolist(), w["head"].tolist(), w["split"].tolist(),
                     w["ntiles"].tolist()))
    assert got == sorted(map(tuple, o.work.tolist()))
    assert np.array_equal(w["stream"], o.tiles[w["tile"], 0])
    # each kind costliest first, the kinds in alternating runs of 256 (groups
    # first) until one runs out
    cost = w["keys"].astype(np.int64) * np.where(w["ntiles"] > 1, 4, 1)
    grp = w["ntiles"] > 1
    for kind in (grp, ~grp):
        c = cost[kind]
        assert all(c[i] >= c[i + 1] for i in range(len(c) - 1))
    ng, n1 = int(grp.sum()), int((~grp).sum())
    expect, i, j = [], 0, 0
    while i < ng or j < n1:
        take = min(256, ng - i)
        expect += [True] * take
        i += take
        take = min(256, n1 - j)
        expect += [False] * take
        j += take
    assert grp.tolist() == expect
    for ti, sp, nt, k in zip(w["tile"], w["split"], w["ntiles"], w["keys"]):
        s, _r0, n, p0 = o.tiles[ti + nt - 1]
        last = o.keys[s] if full else o.keys[s] - o.rows[s] + p0 + n
        lo, hi = o.split_range(s, sp)
        assert k == min(hi, last) - lo > 0
    assert np.array_equal(t["conv_state"], np.array(cs, dtype=np.uint64).ravel())
    assert np.array_equal(t["k"], np.array(kp, dtype=np.uint64).ravel())
    assert np.array_equal(t["v"], np.array(vp, dtype=np.uint64).ravel())


@pytest.mark.parametrize("config", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("full", [False, True])
def test_table_bit_exact_on_workloads(config, full):
    _compare(workloads.streams_for(config), full)


_stream = st.integers(1, 600).flatmap(
    lambda w: st.integers(w, 131072).map(lambda k: (w, k, min(((k + 31) // 32) * 32 + 32 * (k % 3), 131072))))


@settings(max_examples=80, deadline=None)
@given(st.lists(_stream, min_size=1, max_size=12).filter(lambda s: sum(w for w, _, _ in s) <= 2048))
def test_table_bit_exact_random(streams):
    _compare(streams)
    _compare(streams, full=True)


def test_size_query_and_capacity():
    streams = workloads.streams_for(0)
    info, blob, _, (cs, kp, vp) = _build(streams)
    small = np.zeros(int(info.blob_bytes) - 16, dtype=np.uint8)
    with pytest.raises(asv.AsvError) as e:
        asv.seg_table_build(streams, cs, kp, vp, blob=small)
    assert e.value.code == -4
    assert not small.any()  # nothing written on failure


@pytest.mark.parametrize("streams,code", [
    ([(0, 16, 32)], -2), ([(4, 3, 32)], -2), ([(1, 131073, 131104)], -2), ([(1, 64, 32)], -2),
    ([(1, 16, 48)], -2), ([(1, 16, 131104)], -2), ([(16, 32, 32)] * 129, -2),
])
def test_refusals_match_the_oracle(streams, code):
    with pytest.raises(ValueError):
        otable.build(streams)
    with pytest.raises(asv.AsvError) as e:
        _build(streams)
    assert e.value.code == code


def test_refuses_aliasing_and_misaligned_addresses():
    streams = [(1, 100, 128), (2, 100, 128)]
    _, _, _, (cs, kp, vp) = _build(streams)
    # every stream naming the first stream's conv state / kv cache
    with pytest.raises(asv.AsvError) as e:
        asv.seg_table_build(streams, [[cs[0][0], cs[0][0]]], kp, vp)
    assert e.value.code == -1
    with pytest.raises(asv.AsvError) as e:
        asv.seg_table_build(streams, cs, [[kp[0][0], kp[0][0]]], vp)
    assert e.value.code == -1
    with pytest.raises(asv.AsvError) as e:
        asv.seg_table_build(streams, cs, kp, [[vp[0][0], vp[0][0] + 64]])
    assert e.value.code == -1
    with pytest.raises(asv.AsvError) as e:      # a K cache overlapping another stream's V
        asv.seg_table_build(streams, cs, [[kp[0][0], vp[0][0]]], vp)
    assert e.value.code == -1
    with pytest.raises(asv.AsvError) as e:
        asv.seg_table_build(streams, [[cs[0][0] + 8, cs[0][1]]], kp, vp)
    assert e.value.code == -1
    with pytest.raises(asv.AsvError) as e:
        asv.seg_table_build(streams, [[0, cs[0][1]]], kp, vp)
    assert e.value.code == -1


def test_tables_without_layers_and_counts_at_1_32_2048_rows():
    for streams, expect in [([(1, 4096, 4096)], 192), ([(1, 1000, 1024)] * 32, 2048),
                            ([(16, 131072, 131072)] * 128, 128 * 16 * 32 * 19)]:
        info, _ = asv.seg_table_build(streams)
        assert info.n_rows in (1, 32, 2048) and info.partial_count == expect
        assert info.partial_count == otable.build(streams).partial_count


def test_block_table_refuses_what_the_causal_one_refuses():
    bad = [(0, 10, 32)]
    cs = _fake_ptrs([(1, 10, 32)], 1, lambda s: 8192, 1 << 40)
    with pytest.raises(asv.AsvError) as e:
        asv.seg_table_build(bad, cs, [], [], full=True)
    assert e.value.code == -2


def test_draft_ids_refusals_on_the_host():
    for args, code in [((None, -1, None, None, 0, 10, None, 0, None), -2),
                       ((None, 1, None, None, 0, 0, None, 0, None), -2),
                       ((None, 1, None, None, 5, 10, None, 5, None), -1)]:
        with pytest.raises(asv.AsvError) as e:
            asv.draft_ids(*args, stream=0)
        assert e.value.code == code
    asv.draft_ids(None, 0, None, None, 0, 10, None, 0, None, stream=0)


def test_markov_refusals_on_the_host():
    """Every refusal happens before a launch (fake, aligned device addresses)."""
    A = 1 << 20
    ok = dict(base=A, rows=8, row_stride=1000, chains=[(0, 4), (4, 4)], prev0=A, w1=A, w2c=A,
              vocab=1000, rank=64, pick=A, flag=A)
    ws = asv.markov_workspace(1000)
    assert ws == 2 * 4 * 32 * 4      # two halves: a 4-byte record per chain and scan block
    # the larger of the two forms' records: 4 bytes a 256-token block and
    # chain, or 8 bytes a 512-token block and chain (resident)
    for vocab in (1, 255, 256, 257, 512, 513, 131072, 600000):
        launches = 2 * 32 * 4 * -(-vocab // 256)
        resident = 2 * 32 * 8 * -(-vocab // 512)
        assert asv.markov_workspace(vocab) == max(launches, resident), vocab
    assert asv.markov_workspace(0) == 0 and asv.markov_workspace((1 << 30) + 1) == 0

    def call(workspace_bytes=ws, **kw):
        a = dict(ok, **kw)
        L = asv.lib()
        arr = (asv.MarkovChain * max(1, len(a["chains"])))(*[asv.MarkovChain(r, d) for r, d in a["chains"]])
        return L.asv_markov_pick(a["base"], a["rows"], a["row_stride"], arr, len(a["chains"]),
                                 a["prev0"], a["w1"], a["w2c"], a["vocab"], a["rank"], a["pick"],
                                 a["flag"], A, workspace_bytes, 0)

    assert call(rank=12) == -3 and call(rank=264) == -3 and call(rank=0) == -3
    assert call(chains=[(0, 0)]) == -2 and call(chains=[(0, 17)], rows=32) == -2
    assert call(chains=[(0, 4), (3, 2)]) == -2                    # two chains share row 3
    assert call(chains=[(6, 4)]) == -2                            # past the rows
    assert call(chains=[(i, 1) for i in range(33)], rows=40) == -2
    assert call(vocab=0) == -2 and call(row_stride=999) == -2
    assert call(base=None) == -1 and call(w1=A + 8) == -1
    assert call(workspace_bytes=ws - 1) == -4
    assert call(chains=[]) == 0                                   # nothing to do, no launch
    a = dict(ok)
    arr = (asv.MarkovChain * 2)(*[asv.MarkovChain(r, d) for r, d in a["chains"]])
    for form in (-1, 3):                                          # an unknown form
        assert asv.lib().asv_markov_pick_form(a["base"], a["rows"], a["row_stride"], arr, 2, a["prev0"],
                                              a["w1"], a["w2c"], a["vocab"], a["rank"], a["pick"],
                                              a["flag"], A, ws, form, 0) == -1
    assert asv.lib().asv_markov_pack_w2(A, 1000, 12, A * 3, 0) == -3
    assert asv.lib().asv_markov_pack_w2(A, 1000, 64, A + 64, 0) == -1   # overlapping


def test_qk_refusals_on_the_host():
    """theta must be a finite number > 0 (the pages' admission fix), eps
    finite and >= 0; no launch happens for a refused call."""
    streams = [(2, 64, 64)]
    k = [[1 << 20]]
    v = [[1 << 21]]
    info, blob = asv.seg_table_build(streams, [], k, v)
    A = 1 << 24
    L = asv.lib()
    def call(theta=1e6, eps=1e-5, layer=0, qkv=A, q_out=A * 2):
        return L.asv_shared_qk(ctypes.byref(info), A * 3, layer, qkv, A * 4, A * 5, theta, eps, q_out, 0)
    for bad in (float("inf"), float("nan"), 0.0, -1.0, 1e400):
        assert call(theta=bad) == -2
    assert call(eps=-1e-9) == -2 and call(eps=float("nan")) == -2
    assert call(layer=1) == -2 and call(layer=-1) == -2
    assert call(qkv=A + 8) == -1 and call(qkv=None) == -1
    assert call(q_out=A) == -1                                  # q_out overlaps qkv
