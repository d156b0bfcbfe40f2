"""GPU parity of the kernels after the hot path, through the C ABI:
the draft-id gather (bit-exact, with its failure flags)."""

import numpy as np
import pytest
import torch

from oracle import argmax as oargmax
from oracle import draft as odraft

import attention_stream_verify_amd as asv

pytestmark = pytest.mark.gpu

QNAN, POS_INF, NEG_INF = 0x7FC0, 0x7F80, 0xFF80


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def _draft_gpu(spans, pick, flag, vocab, n_ids, fill=-7):
    sp = _dev(np.asarray(spans, dtype=np.int32).reshape(-1, 3), torch.int32)
    p = _dev(pick.astype(np.int32), torch.int32)
    f = _dev(flag.astype(np.uint8), torch.uint8)
    ids = torch.full((n_ids,), fill, dtype=torch.int32, device="cuda")
    fail = torch.full((len(spans),), 9, dtype=torch.uint8, device="cuda")
    asv.draft_ids(sp, len(spans), p, f, len(pick), vocab, ids, n_ids, fail)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), fail.cpu().numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_draft_ids_bit_exact_random(seed):
    rng = np.random.default_rng(seed)
    vocab, n_picks, n_ids = 128000, 300, 400
    pick = rng.integers(0, vocab, n_picks).astype(np.int32)
    bad = rng.random(n_picks) < 0.05
    pick[bad] = rng.choice([-1, vocab, vocab + 5, 2**31 - 1, -(2**31)], bad.sum())
    flag = (rng.random(n_picks) < 0.05).astype(np.uint8)
    # destinations disjoint (each stream owns its window of ids); sources
    # overlap freely; the first span starts before ids, the last runs past it
    spans, cursor = [], -3
    for s in range(44):
        count = int(rng.integers(-2, 12))
        spans.append((int(rng.integers(-3, n_picks)), cursor, count))
        cursor += max(0, count) + int(rng.integers(0, 4))
    spans += [(n_picks - 2, cursor, 6), (0, cursor + 6, 0), (10, n_ids - 3, 1000)]
    assert cursor + 6 < n_ids - 3
    got_ids, got_fail = _draft_gpu(spans, pick, flag, vocab, n_ids)
    ids = np.full(n_ids, -7, dtype=np.int32)
    fail = odraft.draft_ids(spans, pick, flag, vocab, ids)
    assert np.array_equal(got_ids, ids)
    assert np.array_equal(got_fail, fail)


def test_draft_ids_after_row_argmax_with_planted_rows():
    rng = np.random.default_rng(5)
    rows, vocab = 12, 128000
    logits = (rng.standard_normal((rows, vocab)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    logits[2, 99] = QNAN
    logits[5, 1234] = POS_INF
    logits[9, 0] = NEG_INF
    L = _dev(logits.view(np.int16), torch.int16)
    pick = torch.empty(rows, dtype=torch.int32, device="cuda")
    flag = torch.empty(rows, dtype=torch.uint8, device="cuda")
    ws = torch.empty(asv.row_argmax_workspace(rows, vocab), dtype=torch.uint8, device="cuda")
    asv.row_argmax(L, rows, vocab, vocab, pick, flag, ws)
    spans = [(0, 0, 3), (3, 3, 3), (6, 6, 3), (9, 9, 3)]     # four streams of three drafts
    sp = _dev(np.asarray(spans, dtype=np.int32), torch.int32)
    ids = torch.zeros(rows, dtype=torch.int32, device="cuda")
    fail = torch.zeros(4, dtype=torch.uint8, device="cuda")
    asv.draft_ids(sp, 4, pick, flag, rows, vocab, ids, rows, fail)
    torch.cuda.synchronize()
    rp, rf = oargmax.row_argmax(logits)
    ref_ids = np.zeros(rows, dtype=np.int32)
    ref_fail = odraft.draft_ids(spans, rp, rf, vocab, ref_ids)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert fail.cpu().numpy().tolist() == ref_fail.tolist() == [1, 1, 0, 1]


def test_draft_ids_zero_streams():
    asv.draft_ids(None, 0, None, None, 0, 10, None, 0, None)   # launches nothing


# ---- Markov-head step -------------------------------------------------------

from oracle import markov as omarkov  # noqa: E402


def _bf16(rng, shape, scale=1.0):
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(scale)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _markov_gpu(base, chains, prev0, w1, w2, fill_pick=-7, fill_flag=9, form=None):
    rows, vocab = base.shape
    rank = w1.shape[1]
    B = _dev(base.view(np.int16), torch.int16)
    W1 = _dev(w1.view(np.int16), torch.int16)
    W2 = _dev(w2.view(np.int16), torch.int16)
    W2c = torch.empty_like(W2)
    asv.markov_pack_w2(W2, vocab, rank, W2c)
    P0 = _dev(np.asarray(prev0, dtype=np.int32), torch.int32)
    pick = torch.full((rows,), fill_pick, dtype=torch.int32, device="cuda")
    flag = torch.full((rows,), fill_flag, dtype=torch.uint8, device="cuda")
    ws = torch.empty(asv.markov_workspace(vocab), dtype=torch.uint8, device="cuda")
    asv.markov_pick(B, rows, vocab, chains, P0, W1, W2c, vocab, rank, pick, flag, ws, form=form)
    torch.cuda.synchronize()
    return pick.cpu().numpy(), flag.cpu().numpy()


def _markov_ref(base, chains, prev0, w1, w2, fill_pick=-7, fill_flag=9):
    rows = base.shape[0]
    pick = np.full(rows, fill_pick, dtype=np.int32)
    flag = np.full(rows, fill_flag, dtype=np.uint8)
    omarkov.markov_pick(base, chains, prev0, w1, w2, pick, flag)
    return pick, flag


# Both forms of the pass (one launch a depth; one resident launch) on every
# case below; "auto" is what asv_markov_pick takes.
FORMS = ["launches", "resident"]


def _check_markov(base, chains, prev0, w1, w2, form="auto"):
    print(f"markov case ({form}): vocab {base.shape[1]} rank {w1.shape[1]} chains {chains}", flush=True)
    gp, gf = _markov_gpu(base, chains, prev0, w1, w2, form=form)
    rp, rf = _markov_ref(base, chains, prev0, w1, w2)
    assert np.array_equal(gp, rp), (gp, rp)
    assert np.array_equal(gf, rf), (gf, rf)
    return gp, gf


def test_markov_pack_is_the_tiled_layout():
    """Tiles of 64 tokens, each [rank/8][tokens of the tile][8], the last
    tile shorter when 64 does not divide the vocabulary."""
    rng = np.random.default_rng(11)
    for vocab, rank in [(1, 8), (64, 8), (1000, 24), (4099, 256)]:
        w2 = _bf16(rng, (vocab, rank))
        W2 = _dev(w2.view(np.int16), torch.int16)
        W2c = torch.empty_like(W2)
        asv.markov_pack_w2(W2, vocab, rank, W2c)
        torch.cuda.synchronize()
        want = np.concatenate([w2[t:t + 64].reshape(-1, rank // 8, 8).transpose(1, 0, 2).reshape(-1)
                               for t in range(0, vocab, 64)])
        assert np.array_equal(W2c.cpu().numpy().view(np.uint16).reshape(-1), want)


@pytest.mark.parametrize("form", FORMS)
def test_markov_bench_shape_parity(form):
    """The pass the bench times: 4 chains x depth 8 (a hold pass of 32 rows)
    at vocabulary 128,000 and rank 256, weights N(0, 0.3), logits N(0, 3)."""
    rng = np.random.default_rng(20)
    vocab, rank = 128000, 256
    w1, w2 = _bf16(rng, (vocab, rank), 0.3), _bf16(rng, (vocab, rank), 0.3)
    base = _bf16(rng, (32, vocab), 3.0)
    _check_markov(base, [(0, 8), (8, 8), (16, 8), (24, 8)], [17, 4242, 90000, 127999], w1, w2, form)


@pytest.mark.parametrize("form", FORMS + ["auto"])
def test_markov_full_shape_parity(form):
    """vocabulary 128,000, rank 256: three chains of depths 3, 2, 1."""
    rng = np.random.default_rng(12)
    vocab, rank = 128000, 256
    w1, w2 = _bf16(rng, (vocab, rank), 0.3), _bf16(rng, (vocab, rank), 0.3)
    base = _bf16(rng, (6, vocab), 3.0)
    _check_markov(base, [(0, 3), (3, 2), (5, 1)], [17, 127999, 5000], w1, w2, form)


@pytest.mark.parametrize("vocab,rank,chains", [
    (1, 8, [(0, 2)]),
    (7, 16, [(0, 3), (3, 1)]),
    (255, 64, [(1, 2), (4, 3)]),
    (256, 8, [(0, 1)]),
    (257, 256, [(0, 2), (2, 2), (4, 2), (6, 2), (8, 2)]),          # a partial group of four
    (1000, 24, [(i, 1) for i in range(32)]),                          # the most chains
    (2000, 256, [(2 * i, 2) for i in range(32)]),                     # 32 chains folded a depth on
    (4099, 136, [(0, 9), (9, 9), (18, 9)]),                           # the drafter's depth
    (3000, 256, [(0, 16)]),                                           # the longest chain
])
@pytest.mark.parametrize("form", FORMS)
def test_markov_ragged_parity(vocab, rank, chains, form):
    rng = np.random.default_rng(vocab * 7 + rank)
    rows = max(r + d for r, d in chains) + 1
    w1, w2 = _bf16(rng, (vocab, rank), 0.5), _bf16(rng, (vocab, rank), 0.5)
    base = _bf16(rng, (rows, vocab), 2.0)
    prev0 = rng.integers(0, vocab, len(chains))
    gp, gf = _check_markov(base, chains, prev0, w1, w2, form)
    assert gp[-1] == -7 and gf[-1] == 9                               # a row in no chain


def test_markov_large_vocabulary():
    """2,344 scan blocks a depth (vocab 600,000 at rank 8): the fold reads
    its records in several rounds of eight a lane. 1,172 blocks of 512
    tokens are more than the resident form takes: it is refused, and the
    automatic choice runs one launch a depth."""
    rng = np.random.default_rng(15)
    vocab, rank = 600000, 8
    w1, w2 = _bf16(rng, (vocab, rank), 0.5), _bf16(rng, (vocab, rank), 0.5)
    base = _bf16(rng, (4, vocab), 2.0)
    _check_markov(base, [(0, 3)], [123456], w1, w2)
    with pytest.raises(asv.AsvError) as refused:
        _markov_gpu(base, [(0, 3)], [123456], w1, w2, form="resident")
    assert refused.value.code == -3                                   # ASV_E_UNSUPPORTED


@pytest.mark.parametrize("form", FORMS)
def test_markov_largest_resident_vocabulary(form):
    """131,072 tokens at rank 256: 256 blocks of 512, one a CU, the most the
    resident form holds on a 256-CU device (the automatic choice takes it)."""
    rng = np.random.default_rng(16)
    vocab, rank = 131072, 256
    w1, w2 = _bf16(rng, (vocab, rank), 0.3), _bf16(rng, (vocab, rank), 0.3)
    base = _bf16(rng, (5, vocab), 3.0)
    _check_markov(base, [(0, 4), (4, 1)], [131071, 0], w1, w2, form)


@pytest.mark.parametrize("form", FORMS)
def test_markov_most_resident_blocks(form):
    """262,144 tokens at rank 8: 512 blocks of 512, the most the resident
    form takes (several a CU at this rank), so each fold reads eight
    records a lane."""
    rng = np.random.default_rng(18)
    vocab, rank = 262144, 8
    w1, w2 = _bf16(rng, (vocab, rank), 0.5), _bf16(rng, (vocab, rank), 0.5)
    base = _bf16(rng, (6, vocab), 2.0)
    _check_markov(base, [(0, 3), (3, 2)], [262143, 77], w1, w2, form)


def test_markov_resident_back_to_back_calls():
    """Two resident passes in a row on one workspace, the second with fewer
    chains and depths: the records of the first (tags up to its depth) must
    not be taken for the second's."""
    rng = np.random.default_rng(17)
    vocab, rank = 20000, 64
    w1, w2 = _bf16(rng, (vocab, rank), 0.5), _bf16(rng, (vocab, rank), 0.5)
    base = _bf16(rng, (24, vocab), 2.0)
    W1 = _dev(w1.view(np.int16), torch.int16)
    W2 = _dev(w2.view(np.int16), torch.int16)
    W2c = torch.empty_like(W2)
    asv.markov_pack_w2(W2, vocab, rank, W2c)
    B = _dev(base.view(np.int16), torch.int16)
    ws = torch.empty(asv.markov_workspace(vocab), dtype=torch.uint8, device="cuda")
    for chains, prev0 in [([(0, 8), (8, 8), (16, 8)], [5, 6, 7]), ([(3, 2)], [19999])]:
        print(f"markov back to back: chains {chains}", flush=True)
        P0 = _dev(np.asarray(prev0, dtype=np.int32), torch.int32)
        pick = torch.full((24,), -7, dtype=torch.int32, device="cuda")
        flag = torch.full((24,), 9, dtype=torch.uint8, device="cuda")
        asv.markov_pick(B, 24, vocab, chains, P0, W1, W2c, vocab, rank, pick, flag, ws, form="resident")
        torch.cuda.synchronize()
        rp, rf = _markov_ref(base, chains, prev0, w1, w2)
        assert np.array_equal(pick.cpu().numpy(), rp)
        assert np.array_equal(flag.cpu().numpy(), rf)


@pytest.mark.parametrize("form", FORMS)
def test_markov_planted_nonfinite_and_invalid_tokens(form):
    rng = np.random.default_rng(13)
    vocab, rank = 5000, 64
    w1, w2 = _bf16(rng, (vocab, rank), 0.5), _bf16(rng, (vocab, rank), 0.5)
    w2[4500, 5] = POS_INF                               # token 4500's dot is +-Inf or NaN
    base = _bf16(rng, (10, vocab), 2.0)
    base[0, 77] = QNAN
    base[1, 4000] = POS_INF                             # picked, flagged
    base[2, :] = NEG_INF                                # every score -Inf (or NaN at 321)
    base[3, :] = QNAN                                   # no real score: pick 0
    chains = [(0, 4), (4, 2), (6, 2), (8, 2)]
    prev0 = [3, -1, vocab, 2**31 - 1]                   # three invalid first tokens
    gp, gf = _check_markov(base, chains, prev0, w1, w2, form)
    assert gf[[0, 1, 3, 4, 6, 8]].tolist() == [1] * 6
    assert gp[1] == 4000 and gp[3] == 0


@pytest.mark.parametrize("form", FORMS)
def test_markov_subnormal_products(form):
    """Weights near 2^-64: the products lie near or below float32's smallest
    normal 2^-126, so a flush to zero anywhere would change the sums, while
    the sums (near 2^-125) keep enough bf16 steps to tell scores apart."""
    rng = np.random.default_rng(14)
    vocab, rank = 2048, 64
    tiny = 2.0 ** -64
    w1, w2 = _bf16(rng, (vocab, rank), tiny), _bf16(rng, (vocab, rank), tiny)
    base = np.zeros((4, vocab), dtype=np.uint16)
    _check_markov(base, [(0, 4)], [9], w1, w2, form)


@pytest.mark.parametrize("form", FORMS)
def test_markov_ties_go_to_the_lowest_token(form):
    vocab, rank = 3000, 8
    w1 = np.zeros((vocab, rank), dtype=np.uint16)
    w2 = np.zeros((vocab, rank), dtype=np.uint16)
    base = np.zeros((2, vocab), dtype=np.uint16)
    for t in (2999, 1700, 300, 257):                    # equal maxima across blocks
        base[0, t] = 0x4000                             # 2.0
    base[1, :] = 0x8000                                 # -0 everywhere: ties with +0
    base[1, 2500] = 0x0000
    gp, gf = _check_markov(base, [(0, 2)], [1], w1, w2, form)
    assert gp.tolist() == [257, 0] and gf.tolist() == [0, 0]


def test_markov_resident_graph_replays():
    """The resident pass (its clearing launch and the pass itself) captured as
    a HIP graph: every replay, with eager passes of other inputs and
    synchronisations between the replays, gives the oracle's picks and flags
    (the records are cleared by a kernel, not a memset, so each replay starts
    clean)."""
    rng = np.random.default_rng(19)
    vocab, rank = 20000, 64
    w1, w2 = _bf16(rng, (vocab, rank), 0.5), _bf16(rng, (vocab, rank), 0.5)
    base = _bf16(rng, (16, vocab), 2.0)
    chains, prev0 = [(0, 6), (6, 5), (11, 4)], [3, 19999, 1234]
    W1 = _dev(w1.view(np.int16), torch.int16)
    W2 = _dev(w2.view(np.int16), torch.int16)
    W2c = torch.empty_like(W2)
    asv.markov_pack_w2(W2, vocab, rank, W2c)
    B = _dev(base.view(np.int16), torch.int16)
    P0 = _dev(np.asarray(prev0, dtype=np.int32), torch.int32)
    pick = torch.full((16,), -7, dtype=torch.int32, device="cuda")
    flag = torch.full((16,), 9, dtype=torch.uint8, device="cuda")
    ws = torch.empty(asv.markov_workspace(vocab), dtype=torch.uint8, device="cuda")
    rp, rf = _markov_ref(base, chains, prev0, w1, w2)
    # other inputs for the eager passes between replays (the same workspace)
    base2 = _bf16(rng, (16, vocab), 2.0)
    B2 = _dev(base2.view(np.int16), torch.int16)
    rp2, rf2 = _markov_ref(base2, [(2, 7)], prev0[:1], w1, w2)   # chain 0 of P0: token 3
    pick2 = torch.full((16,), -7, dtype=torch.int32, device="cuda")
    flag2 = torch.full((16,), 9, dtype=torch.uint8, device="cuda")

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        asv.markov_pick(B, 16, vocab, chains, P0, W1, W2c, vocab, rank, pick, flag, ws, form="resident")
    for replay in range(4):
        print(f"markov graph replay {replay}", flush=True)
        pick.fill_(-7)
        flag.fill_(9)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(pick.cpu().numpy(), rp), replay
        assert np.array_equal(flag.cpu().numpy(), rf), replay
        asv.markov_pick(B2, 16, vocab, [(2, 7)], P0, W1, W2c, vocab, rank, pick2, flag2, ws, form="resident")
        torch.cuda.synchronize()
        assert np.array_equal(pick2.cpu().numpy(), rp2), replay
        assert np.array_equal(flag2.cpu().numpy(), rf2), replay
