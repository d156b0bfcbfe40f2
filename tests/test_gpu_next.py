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
