"""Draft-id gather with a failure flag (oracle; test infrastructure only).

PR #1391 "lfm2: draft with LiquidAI's DSpark drafter (--drafter)", its
description and the held-draft fix: a new device kernel moves the drafter's
picks for every window into the id array the verify step consumes, an id
past the vocabulary becoming 0; after the fix it also raises a flag, checked
before the caches are committed, so an invalid pick or one from a NaN or
infinite row fails the same way as on the synchronous path. Readings (listed in the design notes):

* a stream s is a span (src_s, dst_s, count_s): picks[src_s + i] goes to
  ids[dst_s + i] for i < count_s; ids outside the spans are not written;
* an id is valid when 0 <= pick < vocab; an invalid one is written as 0;
* fail_s = 1 when any of the stream's picks is invalid or comes from a row
  whose argmax flag is set (a NaN or an infinity in its scores), else 0;
* a span that reaches outside the pick or id arrays fails its stream and
  writes nothing out of range (the entries inside still follow the rules).
"""

import numpy as np


def draft_ids(spans, pick, pick_flag, vocab, ids):
    """spans: [(src, dst, count)]; pick int32 [n_picks]; pick_flag uint8
    [n_picks]; ids int32 [n_ids] (updated in place). Returns fail uint8
    [n_streams]."""
    pick = np.asarray(pick, dtype=np.int64)
    n_picks, n_ids = len(pick), len(ids)
    fail = np.zeros(len(spans), dtype=np.uint8)
    for s, (src, dst, count) in enumerate(spans):
        for i in range(max(0, int(count))):
            a, b = int(src) + i, int(dst) + i
            if not (0 <= a < n_picks and 0 <= b < n_ids):
                fail[s] = 1
                continue
            p = int(pick[a])
            valid = 0 <= p < vocab
            ids[b] = p if valid else 0
            if not valid or pick_flag[a] != 0:
                fail[s] = 1
    return fail
