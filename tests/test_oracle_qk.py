"""Pins of the qk-stage oracle (PR #1377: a qk launch before attention and
merge in every attention layer, run once a layer over every row of a shared
round; PR #1391: the target's RoPE is half-split and takes norm gains; a
rope theta must be finite).

Pinned against: hand-derived cases (tests/golden/qk_hand.json), torch's
rms_norm in float64, RoPE written as a complex multiplication, RoPE's
relative-position property, and hand-checked row positions and cache
placement."""

import json
import os

import numpy as np
import torch

from oracle import bf16, qk

HERE = os.path.dirname(__file__)


def rand_bf16(rng, shape, scale=1.0):
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(scale)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_hand_cases():
    g = json.load(open(os.path.join(HERE, "golden", "qk_hand.json")))
    for case in g["cases"]:
        x = np.zeros((1, 64))
        for i, v in case["x"].items():
            x[0, int(i)] = v
        out = qk.norm_rope(x, np.ones(64), case["pos"], g["theta"], g["eps"])
        got = bf16.to_f64(bf16.round_f64(out))[0]
        want = np.zeros(64)
        for i, v in case["out"].items():
            want[int(i)] = v
        assert np.array_equal(got, want), case["derivation"]


def test_norm_is_torch_rms_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 64)) * 3
    g = rng.standard_normal(64)
    for eps in (0.0, 1e-6, 1e-5):
        want = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), weight=torch.from_numpy(g),
                                            eps=eps).numpy()
        assert np.allclose(qk.norm_rope(x, g, 0, 1e6, eps), want, rtol=1e-13, atol=1e-13)


def test_rope_is_a_complex_rotation():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 64))
    g = rng.standard_normal(64)
    for theta, pos in ((1e6, 131071), (10000.0, 5), (500000.0, 65536)):
        y = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), weight=torch.from_numpy(g),
                                         eps=1e-5).numpy()
        freq = theta ** (-np.arange(32) / 32.0)
        z = (y[:, :32] + 1j * y[:, 32:]) * np.exp(1j * pos * freq)
        want = np.concatenate([z.real, z.imag], axis=1)
        assert np.allclose(qk.norm_rope(x, g, pos, theta, 1e-5), want, rtol=1e-9, atol=1e-9)


def test_scores_depend_on_the_position_difference_only():
    rng = np.random.default_rng(3)
    q, k, g = rng.standard_normal(64), rng.standard_normal(64), rng.standard_normal(64)
    theta, eps = 1e6, 1e-5
    base = qk.norm_rope(q, g, 1000, theta, eps) @ qk.norm_rope(k, g, 990, theta, eps)
    for t in (1, 77, 100000):
        moved = qk.norm_rope(q, g, 1000 + t, theta, eps) @ qk.norm_rope(k, g, 990 + t, theta, eps)
        assert abs(moved - base) <= 1e-9 * max(1.0, abs(base))
    other = qk.norm_rope(q, g, 1000, theta, eps) @ qk.norm_rope(k, g, 980, theta, eps)
    assert abs(other - base) > 1e-6


def test_positions_by_hand():
    st, pos = qk.positions([(2, 10, 32), (1, 5, 32), (3, 3, 64)])
    assert st.tolist() == [0, 0, 1, 2, 2, 2]
    assert pos.tolist() == [8, 9, 4, 0, 1, 2]


def test_rows_and_append():
    rng = np.random.default_rng(4)
    streams = [(2, 40, 64), (1, 33, 64)]
    qkv = rand_bf16(rng, (3, qk.QKV))
    gq, gk = rand_bf16(rng, 64), rand_bf16(rng, 64)
    Q, Kn, Vn, st, pos = qk.qk_rows(streams, qkv, gq, gk, 1e6, 1e-5)
    # q head 5 of row 1 and k head 3 of row 2, by the definition above
    x = bf16.to_f64(qkv[1, 5 * 64:6 * 64])
    assert np.array_equal(Q[1, 5], bf16.round_f64(qk.norm_rope(x, bf16.to_f64(gq), 39, 1e6, 1e-5)))
    x = bf16.to_f64(qkv[2, 32 * 64 + 3 * 64:32 * 64 + 4 * 64])
    assert np.array_equal(Kn[2, 3], bf16.round_f64(qk.norm_rope(x, bf16.to_f64(gk), 32, 1e6, 1e-5)))
    assert np.array_equal(Vn[2, 7], qkv[2, 40 * 64 + 7 * 64:40 * 64 + 8 * 64])      # v copied
    K = [rand_bf16(rng, (8, 64, 64)) for _ in streams]
    V = [rand_bf16(rng, (8, 64, 64)) for _ in streams]
    K2, V2 = qk.append(K, V, st, pos, Kn, Vn)
    for s, (w, keys, _cap) in enumerate(streams):
        win = np.zeros(64, dtype=bool)
        win[keys - w:keys] = True
        assert np.array_equal(K2[s][:, ~win], K[s][:, ~win]) and np.array_equal(V2[s][:, ~win], V[s][:, ~win])
    assert np.array_equal(K2[0][:, 38], Kn[0]) and np.array_equal(K2[0][:, 39], Kn[1])
    assert np.array_equal(V2[1][:, 32], Vn[2])
