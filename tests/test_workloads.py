"""The seeded input generators: shapes, layouts, poison and determinism (CPU)."""

import numpy as np
import torch

import workloads
from oracle import argmax, bf16, table


def test_stream_shapes_match_the_workload_recipes():
    s0 = workloads.streams_for(0)
    assert [(w, k) for w, k, _ in s0] == [(1, 16), (2, 64), (3, 128), (4, 256)]
    s1 = workloads.streams_for(1)
    assert len(s1) == 16 and all(w == 1 and 512 <= k <= 4096 for w, k, _ in s1)
    s2 = workloads.streams_for(2)
    assert len(s2) == 16 and all(w == 8 and 2048 <= k <= 32768 for w, k, _ in s2)
    s3 = workloads.streams_for(3)
    assert [k for _, k, _ in s3] == [65536, 98304, 130816, 131072]
    s4 = workloads.streams_for(4)
    assert sum(w for w, _, _ in s4) == 2048
    assert all(1 <= w <= 16 for w, _, _ in s4[:48]) and all(w <= 512 for w, _, _ in s4[48:])
    for ss in (s0, s1, s2, s3, s4):
        table.validate(ss)
        assert all(cap % 256 == 0 and k <= cap <= 131072 for _, k, cap in ss)


def test_v_layout_roundtrip_and_position():
    v = torch.arange(2 * 64 * 64, dtype=torch.int16).reshape(2, 64, 64)
    blk = workloads.v_blocked(v)
    assert blk.shape == (2, 2, 64, 32)
    # key j, dim d of head h sits at [h][j // 32][d][j % 32]
    assert blk[1, 1, 5, 7].item() == v[1, 32 + 7, 5].item()
    assert torch.equal(workloads.v_logical(blk), v)


def test_round_is_seeded_and_poisoned():
    a = workloads.Round(0, "cpu")
    b = workloads.Round(0, "cpu")
    assert torch.equal(a.logits, b.logits) and torch.equal(a.attn[0][0], b.attn[0][0])
    Q, ks, vs = a.attn[0]
    for (w, k, cap), K, V in zip(a.streams, ks, vs):
        kb = K.numpy().view(np.uint16)
        assert bf16.is_nan_bits(kb[:, k:]).all() and not bf16.is_nan_bits(kb[:, :k]).any()
        vl = workloads.v_logical(V).numpy().view(np.uint16)
        assert bf16.is_nan_bits(vl[:, k:]).all() and not bf16.is_nan_bits(vl[:, :k]).any()


def test_tiny_logits_plants():
    a = workloads.Round(0, "cpu")
    L = a.logits.numpy().view(np.uint16)
    pick, flag = argmax.row_argmax(L)
    assert flag.sum() == 1
    ties = [n for n in a.notes if n[0] == "tie"]
    assert len(ties) >= 9
    for _, r, hi, lo in ties:
        if flag[r]:
            continue
        assert pick[r] == min(hi, lo)


def test_logit_plants_on_every_workload_small_vocab():
    g = torch.Generator().manual_seed(5)
    for config, R in [(0, 10), (1, 16), (2, 128), (3, 64), (4, 2048)]:
        L, notes = workloads.logits_for(config, R, g, "cpu", vocab=1000)
        assert L.shape == (R, 1000)
        pick, flag = argmax.row_argmax(L.numpy().view(np.uint16))
        expect_flags = {0: 1, 1: 0, 2: 2, 3: 0, 4: 8}[config]
        assert int(flag.sum()) == expect_flags
