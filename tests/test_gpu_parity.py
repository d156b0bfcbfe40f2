"""GPU parity of the HIP path against the oracle, through the C ABI.

Bit-exact: argmax picks and flags, new conv states. Within the bounds of
tests/helpers.py: conv outputs, attention partials and merged outputs.
Every workload runs at its full size, in the launch configuration the bench
times; where the oracle would take minutes (long contexts, 2,048 rows) it
checks sampled rows, computed one by one.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import argmax as oargmax
from oracle import conv as oconv
from oracle import table as otable

from helpers import (check_attention_layer, check_bf16_out, chunk_rows, host_u16, run_round,
                     sample_rows, sample_rows_every_tile)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    import attention_stream_verify_amd as asv
    asv.lib()
    torch.cuda.init()


def _round(config, **kw):
    print(f"\n[parity] workload {config} {workloads.NAMES[config]} {kw}", flush=True)
    return workloads.Round(config, device="cuda", **kw)


# ------------------------------------------------------------------- argmax

@pytest.mark.parametrize("config", [0, 1, 2, 3, 4])
def test_argmax_bit_exact(config):
    rnd = _round(config, n_conv=0, n_attn=0)
    import attention_stream_verify_amd as asv
    R, V = rnd.logits.shape
    pick = torch.empty(R, dtype=torch.int32, device="cuda")
    flag = torch.empty(R, dtype=torch.uint8, device="cuda")
    ws = torch.empty(asv.row_argmax_workspace(R, V), dtype=torch.uint8, device="cuda")
    asv.row_argmax(rnd.logits, R, V, V, pick, flag, ws)
    torch.cuda.synchronize()
    ep, ef = oargmax.row_argmax(host_u16(rnd.logits))
    assert np.array_equal(pick.cpu().numpy(), ep)
    assert np.array_equal(flag.cpu().numpy(), ef)
    if config in (0, 2, 4):
        assert ef.any()


def _argmax_dev(bits, vocab=None, stride=None):
    import attention_stream_verify_amd as asv
    bits = np.asarray(bits, dtype=np.uint16)
    R, Vw = bits.shape
    vocab = Vw if vocab is None else vocab
    stride = Vw if stride is None else stride
    L = torch.from_numpy(bits.view(np.int16).copy()).cuda()
    pick = torch.full((max(R, 1),), -7, dtype=torch.int32, device="cuda")
    flag = torch.full((max(R, 1),), 9, dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(16, asv.row_argmax_workspace(R, vocab)), dtype=torch.uint8, device="cuda")
    asv.row_argmax(L, R, vocab, stride, pick, flag, ws)
    torch.cuda.synchronize()
    return pick.cpu().numpy()[:R], flag.cpu().numpy()[:R]


@pytest.mark.parametrize("vocab", [1, 7, 8, 9, 8191, 8192, 8193, 16385, 128000])
def test_argmax_ragged_vocab(vocab):
    rng = np.random.default_rng(vocab)
    x = (rng.standard_normal((5, vocab)) * 3).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if vocab > 1:
        bits[1, vocab - 1] = 0x7F80          # +Inf in the ragged tail
        bits[2, :] = bits[2, vocab // 2]      # all equal
        bits[3, :] = 0x7FC0                   # all NaN
        bits[4, 0] = 0x8000                   # -0 vs +0 at the front
        bits[4, 1:] = 0xFF80
    stride = -(-vocab // 8) * 8              # row stride: a multiple of 8 elements
    padded = np.full((5, stride), 0x7F80, dtype=np.uint16)   # +Inf padding is never read
    padded[:, :vocab] = bits
    p, f = _argmax_dev(padded, vocab=vocab, stride=stride)
    ep, ef = oargmax.row_argmax(bits)
    assert np.array_equal(p, ep) and np.array_equal(f, ef)


def test_argmax_ties_across_chunk_boundaries_and_stride():
    V, stride = 20000, 20008
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((6, stride)) * 3).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    big = 0x4300  # 128.0, above every N(0,3) draw
    bits[0, [8191, 8192]] = big               # tie across the first chunk boundary
    bits[1, [16383, 8192, 16384]] = big
    bits[2, [19999, 12000]] = big
    bits[3, V:] = 0x7F80                      # +Inf past vocab: never read
    bits[4, [5, 9000]] = [0x8000, 0x0000]     # -0 and +0 tie ...
    bits[4, :5] = 0xFF80
    bits[4, 6:9000] = 0xFF80
    bits[4, 9001:] = 0xFF80
    bits[5, 100] = 0x7FC0
    p, f = _argmax_dev(bits, vocab=V, stride=stride)
    ep, ef = oargmax.row_argmax(bits[:, :V])
    assert np.array_equal(p, ep) and np.array_equal(f, ef)
    assert p[0] == 8191 and p[1] == 8192 and p[2] == 12000 and f[3] == 0 and p[4] == 5


def test_argmax_zero_rows_and_refusals():
    import attention_stream_verify_amd as asv
    p, f = _argmax_dev(np.zeros((0, 64), dtype=np.uint16))
    assert p.size == 0
    L = torch.zeros((2, 64), dtype=torch.int16, device="cuda")
    pick = torch.zeros(2, dtype=torch.int32, device="cuda")
    flag = torch.zeros(2, dtype=torch.uint8, device="cuda")
    ws = torch.empty(asv.row_argmax_workspace(2, 64), dtype=torch.uint8, device="cuda")
    for args, code in [((2, 64, 60), -2), ((2, 64, 66), -1), ((2, 0, 64), -2)]:
        with pytest.raises(asv.AsvError) as e:
            asv.row_argmax(L, *args, pick, flag, ws)
        assert e.value.code == code
    with pytest.raises(asv.AsvError) as e:
        asv.row_argmax(L, 2, 64, 64, pick, flag, ws[:8])
    assert e.value.code == -4


def test_argmax_planted_controls_go_red():
    """A ties-to-highest expectation and a cleared flag must disagree with the GPU."""
    rnd = _round(0, n_conv=0, n_attn=0)
    bits = host_u16(rnd.logits)
    p, f = _argmax_dev(bits)
    ep, ef = oargmax.row_argmax(bits)
    assert np.array_equal(p, ep) and np.array_equal(f, ef)
    # the same scan taking the LAST maximum (a tie to the highest id)
    hi = np.array([len(r) - 1 - oargmax.row_argmax(r[::-1][None, :])[0][0] for r in bits])
    assert not np.array_equal(p, hi)
    cleared = ef.copy()
    cleared[np.flatnonzero(ef)[0]] = 0
    assert not np.array_equal(f, cleared)


# --------------------------------------------------------------------- conv

@pytest.mark.parametrize("config", [0, 1, 2, 3, 4])
def test_conv_parity(config):
    rnd = _round(config, n_conv=1, n_attn=0, with_logits=False)
    X, W, states = rnd.conv[0]
    before = [host_u16(s) for s in states]
    _, out = run_round(rnd, with_argmax=False)
    t = otable.build(rnd.streams)
    y_ref, st_ref = oconv.shared_conv(t, host_u16(X), host_u16(W), before)
    check_bf16_out(host_u16(out["y"][0]), y_ref, f"conv {config}")
    for s, st in enumerate(states):
        assert np.array_equal(host_u16(st), st_ref[s]), f"state of stream {s}"


@pytest.mark.parametrize("streams", [
    [(1, 40, 64), (2, 40, 64), (3, 40, 64), (4, 40, 64)],            # state only, state + tail rows
    [(15, 100, 128), (16, 100, 128), (17, 100, 128), (33, 100, 128)],  # ragged tiles and one-row tiles
])
def test_conv_parity_ragged_windows(streams):
    """Each stream's first block (state in, last rows for the new state) and
    the blocks past it (history recomputed from the rows before), at window
    sizes around the two-row block and the 16-row tile."""
    rnd = workloads.Round(0, "cuda", n_conv=1, n_attn=0, streams=streams, with_logits=False)
    X, W, states = rnd.conv[0]
    before = [host_u16(s) for s in states]
    _, out = run_round(rnd, with_argmax=False)
    t = otable.build(streams)
    y_ref, st_ref = oconv.shared_conv(t, host_u16(X), host_u16(W), before)
    check_bf16_out(host_u16(out["y"][0]), y_ref, f"conv {streams}")
    for s, st in enumerate(states):
        assert np.array_equal(host_u16(st), st_ref[s]), f"state of stream {s}"


def test_conv_window_equals_one_row_rounds():
    """A window of w rows equals w one-row rounds carried through the state."""
    import attention_stream_verify_amd as asv
    streams = [(5, 64, 64), (1, 32, 32), (17, 100, 128)]
    rnd = workloads.Round(0, "cuda", n_conv=1, n_attn=0, streams=streams, with_logits=False)
    X, W, states = rnd.conv[0]
    st_win = [s.clone() for s in states]
    st_step = [s.clone() for s in states]
    rb = asv.RoundBuffers(streams, [st_win], [], [])
    rb.upload()
    rb.conv(0, X, W)
    y_win = rb.y.clone()
    off = np.cumsum([0] + [w for w, _, _ in streams])
    for s, (w, k, cap) in enumerate(streams):
        for i in range(w):
            one = asv.RoundBuffers([(1, k - w + i + 1, cap)], [[st_step[s]]], [], [])
            one.upload()
            one.conv(0, X[off[s] + i:off[s] + i + 1].contiguous(), W)
            torch.cuda.synchronize()
            assert torch.equal(one.y[0], y_win[off[s] + i])
        assert torch.equal(st_step[s], st_win[s])


# ---------------------------------------------------------------- attention

def _parity_rows(t, config):
    """Every row of the tiny, decode, verify and long-context rounds; at 2,048
    rows, rows from every segment and every 16-row tile of the prompt chunks."""
    return list(range(t.n_rows)) if config != 4 else sample_rows_every_tile(t, 10, config)


def _check_layer_by_part(rnd, rb, out, t, rows, what, full=False):
    """Check window rows and prompt-chunk rows apart and print both."""
    chunk = chunk_rows(t, rows)
    window = [r for r in rows if r not in set(chunk)]
    for part, rr in (("window", window), ("chunk", chunk)):
        if not rr:
            continue
        prel, oerr = check_attention_layer(rnd, rb, out["partials"][0], out["o"][0], 0, rr,
                                           f"{what} {part} rows", full=full)
        print(f"[parity] {what}: {len(rr)} {part} rows (keys {int(t.row_nkeys[rr].min())}-"
              f"{int(t.row_nkeys[rr].max())}), partial o rel err {prel:.2e}, "
              f"output abs err {oerr:.2e}", flush=True)
        if part == "chunk":
            print(f"[parity] {what}: chunk rows checked {rr}", flush=True)


@pytest.mark.parametrize("config", [0, 1, 2, 3, 4])
def test_attention_parity(config):
    rnd = _round(config, n_conv=0, n_attn=1, with_logits=False)
    rb, out = run_round(rnd, with_argmax=False)
    t = otable.build(rnd.streams)
    _check_layer_by_part(rnd, rb, out, t, _parity_rows(t, config), f"attn {config}")


def _edge_rows(t):
    """Rows of every tile (each wave of every group item), except for the
    2,048-row, 131,072-key case, where the oracle would take minutes over
    them: its first and last rows and 24 seeded ones there."""
    if int(t.keys.sum()) * t.n_rows > 100_000_000:
        return sample_rows(t, 24, 5)
    return sample_rows_every_tile(t, 24, 5)


@pytest.mark.parametrize("streams", [
    [(1, 1, 32)],                                # one key
    [(16, 16, 32)],                              # window = whole cache
    [(3, 40, 64), (16, 4097, 4128), (9, 2049, 2080), (2, 513, 544)],   # ragged splits
    [(33, 600, 640), (1, 5000, 5024)],           # a 3-tile chunk
    [(512, 3000, 3072)],                         # a prompt chunk of 32 tiles
    [(16, 7169, 7200)],                          # two split sizes: 4,000 then 3,169 keys
    [(17, 20000, 20000)],                        # 5,568 x 2 then 4,448 x 2; a one-row second tile
    [(16, 14337, 14368), (24, 21505, 21536)],    # 3 and 5 splits, the last one short
    [(2048, 131072, 131072)],                    # both maxima: 2,048 rows, 131,072 keys
    [(64, 100, 128), (100, 150, 160)],           # groups of 4 and 3 tiles, fewer sub-blocks than ring slots
    [(96, 9000, 9024)],                          # 6 tiles: a group of 4, then one of 2
    [(80, 5000, 5024), (1, 40, 64)],             # 5 tiles: a group of 4, then a lone tile
    [(17, 17, 32), (31, 31, 32), (20, 40, 64)],  # groups of one or two sub-blocks, a one-row last tile
])
def test_attention_edge_shapes(streams):
    rnd = workloads.Round(0, "cuda", n_conv=0, n_attn=1, streams=streams, with_logits=False)
    print(f"\n[parity] attention edge {streams}", flush=True)
    rb, out = run_round(rnd, with_argmax=False)
    t = otable.build(streams)
    rows = list(range(t.n_rows)) if t.n_rows <= 64 else _edge_rows(t)
    check_attention_layer(rnd, rb, out["partials"][0], out["o"][0], 0, rows, f"edge {streams}")


# --------------------------------------------------------------- invariants

def _slice_round(rnd, s):
    """Stream s of a round on its own: its rows, its caches, a copy of its state."""
    w, k, cap = rnd.streams[s]
    off = sum(x[0] for x in rnd.streams[:s])
    one = workloads.Round.__new__(workloads.Round)
    one.config, one.seed, one.streams = rnd.config, rnd.seed, [rnd.streams[s]]
    one.n_conv, one.n_attn, one.R, one.S = rnd.n_conv, rnd.n_attn, w, 1
    one.conv = [(X[off:off + w].contiguous(), W, [st[s]]) for (X, W, st) in rnd.conv]
    one.attn = [(Q[off:off + w].contiguous(), [ks[s]], [vs[s]]) for (Q, ks, vs) in rnd.attn]
    one.logits, one.notes = None, []
    return one, off


@pytest.mark.parametrize("config", [0, 2, 4])
def test_shared_round_equals_each_stream_alone(config):
    rnd = _round(config, n_conv=1, n_attn=1, with_logits=False)
    st0 = [s.clone() for s in rnd.conv[0][2]]
    rb, out = run_round(rnd, with_argmax=False)
    shared_states = [s.clone() for s in rnd.conv[0][2]]
    for i, s in enumerate(rnd.conv[0][2]):
        s.copy_(st0[i])                                # rewind the states
    t = otable.build(rnd.streams)
    P = int(rb.info.partial_count)
    po = out["partials"][0][:P * 64].view(P, 64)
    pml = out["partials"][0][P * 64:].view(P, 2)
    # config 4: some windows and every prompt chunk (48-51: 512, 512, 512 and 40 rows)
    streams = range(len(rnd.streams)) if config != 4 else [0, 1, 2, 47, 48, 49, 50, 51]
    for s in streams:
        one, off = _slice_round(rnd, s)
        rb1, out1 = run_round(one, with_argmax=False)
        w = rnd.streams[s][0]
        assert torch.equal(out1["y"][0], out["y"][0][off:off + w])
        assert torch.equal(one.conv[0][2][0], shared_states[s])
        assert torch.equal(out1["o"][0], out["o"][0][off:off + w])
        t1 = otable.build([rnd.streams[s]])
        P1 = int(rb1.info.partial_count)
        po1 = out1["partials"][0][:P1 * 64].view(P1, 64)
        pml1 = out1["partials"][0][P1 * 64:].view(P1, 2)
        for i in range(w):
            for sp in range(t1.row_nsplit(i)):
                a = [t.record(off + i, h, sp) for h in range(32)]
                b = [t1.record(i, h, sp) for h in range(32)]
                assert torch.equal(po[a], po1[b]) and torch.equal(pml[a], pml1[b])


def test_isolation_by_perturbation_and_determinism():
    rnd = _round(2, n_conv=1, n_attn=1, with_logits=False)
    st0 = [s.clone() for s in rnd.conv[0][2]]
    _, base = run_round(rnd, with_argmax=False)
    base_states = [s.clone() for s in rnd.conv[0][2]]
    # determinism: the same inputs give the same bits
    for i, s in enumerate(rnd.conv[0][2]):
        s.copy_(st0[i])
    _, again = run_round(rnd, with_argmax=False)
    for key in ("y", "o", "partials"):
        assert torch.equal(base[key][0], again[key][0])
    # perturb stream 3 everywhere; every other stream keeps its bits
    j, off = 3, sum(w for w, _, _ in rnd.streams[:3])
    w = rnd.streams[j][0]
    X, W, states = rnd.conv[0]
    Q, ks, vs = rnd.attn[0]
    for i, s in enumerate(states):
        s.copy_(st0[i])
    gen = torch.Generator(device="cuda").manual_seed(77)
    X[off:off + w] = torch.randn(X[off:off + w].shape, generator=gen, device="cuda").to(
        torch.bfloat16).view(torch.int16)
    states[j].fill_(0x3F80)
    Q[off:off + w] = torch.randn(Q[off:off + w].shape, generator=gen, device="cuda").to(
        torch.bfloat16).view(torch.int16)
    ks[j].fill_(0x4000)
    vs[j].fill_(0x7FC0)                               # NaN everywhere in stream 3's V
    _, pert = run_round(rnd, with_argmax=False)
    R = sum(x[0] for x in rnd.streams)
    others = np.r_[0:off, off + w:R]
    assert torch.equal(pert["y"][0][others], base["y"][0][others])
    assert torch.equal(pert["o"][0][others], base["o"][0][others])
    for s in range(len(rnd.streams)):
        if s != j:
            assert torch.equal(states[s], base_states[s])
    assert torch.isnan(pert["o"][0][off:off + w].view(torch.bfloat16).float()).all()


# ---------------------------------------------------------- block attention
# Tables from asv_block_table_build: every row sees all of its stream's keys
# (PR #1391's FULL block attention); same kernels, same bounds.

@pytest.mark.parametrize("config", [0, 2, 3, 4])
def test_block_attention_parity(config):
    rnd = _round(config, n_conv=0, n_attn=1, with_logits=False)
    rb, out = run_round(rnd, with_argmax=False, full=True)
    t = otable.build(rnd.streams, full=True)
    _check_layer_by_part(rnd, rb, out, t, _parity_rows(t, config), f"block {config}", full=True)


@pytest.mark.parametrize("streams", [
    [(1, 1, 32)],                                # one key
    [(16, 16, 32)],                              # window = whole cache
    [(3, 40, 64), (16, 4097, 4128), (9, 2049, 2080), (2, 513, 544)],   # ragged splits
    [(33, 600, 640), (1, 5000, 5024)],           # a 3-tile chunk
    [(512, 3000, 3072)],                         # a prompt chunk of 32 tiles
    [(16, 7169, 7200)],                          # two split sizes: 4,000 then 3,169 keys
    [(17, 20000, 20000)],                        # 5,568 x 2 then 4,448 x 2; a one-row second tile
    [(16, 14337, 14368), (24, 21505, 21536)],    # 3 and 5 splits, the last one short
    [(64, 100, 128), (100, 150, 160)],           # groups of 4 and 3 tiles, fewer sub-blocks than ring slots
    [(96, 9000, 9024)],                          # 6 tiles: a group of 4, then one of 2
    [(17, 17, 32), (31, 31, 32), (20, 40, 64)],  # groups of one or two sub-blocks, a one-row last tile
])
def test_block_attention_edge_shapes(streams):
    rnd = workloads.Round(0, "cuda", n_conv=0, n_attn=1, streams=streams, with_logits=False)
    print(f"\n[parity] block attention edge {streams}", flush=True)
    rb, out = run_round(rnd, with_argmax=False, full=True)
    t = otable.build(streams, full=True)
    rows = list(range(t.n_rows)) if t.n_rows <= 64 else _edge_rows(t)
    check_attention_layer(rnd, rb, out["partials"][0], out["o"][0], 0, rows,
                          f"block edge {streams}", full=True)


@pytest.mark.parametrize("config", [2, 4])
def test_block_shared_round_equals_each_stream_alone(config):
    rnd = _round(config, n_conv=0, n_attn=1, with_logits=False)
    rb, out = run_round(rnd, with_argmax=False, full=True)
    t = otable.build(rnd.streams, full=True)
    P = int(rb.info.partial_count)
    po = out["partials"][0][:P * 64].view(P, 64)
    pml = out["partials"][0][P * 64:].view(P, 2)
    streams = range(len(rnd.streams)) if config != 4 else [0, 1, 47, 48, 49, 50, 51]
    for s in streams:
        one, off = _slice_round(rnd, s)
        rb1, out1 = run_round(one, with_argmax=False, full=True)
        w = rnd.streams[s][0]
        assert torch.equal(out1["o"][0], out["o"][0][off:off + w])
        t1 = otable.build([rnd.streams[s]], full=True)
        P1 = int(rb1.info.partial_count)
        po1 = out1["partials"][0][:P1 * 64].view(P1, 64)
        pml1 = out1["partials"][0][P1 * 64:].view(P1, 2)
        for i in range(w):
            for sp in range(t1.row_nsplit(i)):
                a = [t.record(off + i, h, sp) for h in range(32)]
                b = [t1.record(i, h, sp) for h in range(32)]
                assert torch.equal(po[a], po1[b]) and torch.equal(pml[a], pml1[b])
