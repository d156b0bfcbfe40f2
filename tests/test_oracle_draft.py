"""Pins of the draft-id gather oracle (PR #1391: each pick copied exactly or
0 past the vocabulary; a failure flag for NaN, Inf or invalid picks, with
planted controls on both paths)."""

import numpy as np

from oracle import argmax as oargmax
from oracle import draft

POS_INF, NEG_INF, QNAN = 0x7F80, 0xFF80, 0x7FC0


def test_hand_case():
    pick = np.array([5, 7, 128000, -1, 3, 9, 0, 127999], dtype=np.int32)
    flag = np.array([0, 0, 0, 0, 1, 0, 0, 0], dtype=np.uint8)
    ids = np.full(12, -5, dtype=np.int32)
    spans = [(0, 1, 2),        # 5, 7 -> ids 1..2, clean
             (2, 4, 2),        # past the vocabulary and negative -> 0, 0, fails
             (4, 7, 1),        # a flagged row's pick: copied, fails
             (5, 9, 0),        # empty: nothing, clean
             (6, 10, 2)]       # 0 and the last id: clean
    fail = draft.draft_ids(spans, pick, flag, 128000, ids)
    assert fail.tolist() == [0, 1, 1, 0, 0]
    assert ids.tolist() == [-5, 5, 7, -5, 0, 0, -5, 3, -5, -5, 0, 127999]


def test_out_of_range_span_fails_and_writes_inside_only():
    pick = np.array([1, 2, 3], dtype=np.int32)
    flag = np.zeros(3, dtype=np.uint8)
    ids = np.full(4, -1, dtype=np.int32)
    fail = draft.draft_ids([(1, 2, 5)], pick, flag, 10, ids)
    assert fail.tolist() == [1]
    assert ids.tolist() == [-1, -1, 2, 3]


def test_planted_controls_through_the_argmax():
    """Rows with a NaN, +Inf or -Inf logit give flagged picks; their stream
    fails, while a clean stream keeps its exact picks."""
    rng = np.random.default_rng(3)
    vocab = 1000
    logits = (rng.standard_normal((6, vocab)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    logits[1, 17] = QNAN
    logits[3, 400] = POS_INF
    logits[4, 2] = NEG_INF
    pick, flag = oargmax.row_argmax(logits)
    assert flag.tolist() == [0, 1, 0, 1, 1, 0]
    ids = np.zeros(6, dtype=np.int32)
    fail = draft.draft_ids([(0, 0, 1), (1, 1, 1), (2, 2, 1), (3, 3, 1), (4, 4, 1), (5, 5, 1)],
                           pick, flag, vocab, ids)
    assert fail.tolist() == [0, 1, 0, 1, 1, 0]
    assert ids[3] == 400                      # +Inf is a legal maximum: copied, still flagged
    # the clean rows' ids are the argmax picks themselves
    assert [int(ids[r]) for r in (0, 2, 5)] == [int(pick[r]) for r in (0, 2, 5)]
