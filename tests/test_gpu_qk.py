"""GPU parity of the qk stage through the C ABI (asv_shared_qk): q and k
head norm + half-split RoPE, and the window's K/V appended to every stream's
cache, on every workload's rows at full size.

Bound: the kernel forms the angles in float64 and runs the norm and the
rotation in float32, so an output lies within one bf16 step of the float64
value, plus a float32 slack of 2^-18 times the head's largest |y| where the
rotation cancels. V is copied, so it is compared bit for bit, and every
cache entry outside the windows must keep its bits."""

import numpy as np
import pytest
import torch

import attention_stream_verify_amd as asv
import workloads
from oracle import bf16 as obf16
from oracle import qk as oqk

pytestmark = pytest.mark.gpu


def _u16(t):
    return t.detach().cpu().numpy().view(np.uint16)


def _ulp(v):
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _check_heads(got_bits, x_heads, gain, pos, what):
    exact = oqk.norm_rope(x_heads, gain, pos, workloads.ROPE_THETA, workloads.NORM_EPS)
    g = obf16.to_f64(got_bits)
    y = oqk.norm_rope(x_heads, gain, 0, workloads.ROPE_THETA, workloads.NORM_EPS)
    slack = 2.0 ** -18 * np.abs(y).max(axis=-1, keepdims=True)
    err = np.abs(g - exact)
    bad = err > _ulp(exact) + slack
    assert not bad.any(), f"{what}: {int(bad.sum())} outside, max err {err.max():.3e}"
    return float(np.mean(obf16.round_f64(exact) == got_bits))


@pytest.mark.parametrize("config", [0, 1, 2, 3, 4])
def test_qk_parity(config):
    print(f"qk parity: workload {workloads.NAMES[config]}", flush=True)
    rnd = workloads.Round(config, device="cuda", n_conv=0, n_attn=1, with_logits=False)
    qkv, gq, gk = workloads.qk_inputs(rnd.R, seed=1000 + config, device="cuda")
    K, V = rnd.attn[0][1], rnd.attn[0][2]
    K0 = [_u16(k) for k in K]
    V0 = [_u16(workloads.v_logical(v)) for v in V]
    rb = asv.RoundBuffers(rnd.streams, [], [K], [V], device="cuda")
    rb.upload()
    rb.qk(0, qkv, gq, gk, workloads.ROPE_THETA, workloads.NORM_EPS)
    torch.cuda.synchronize()
    Qg = _u16(rb.q)
    K1 = [_u16(k) for k in K]
    V1 = [_u16(workloads.v_logical(v)) for v in V]

    qkv_h, gq_h, gk_h = _u16(qkv), _u16(gq), _u16(gk)
    _, _, Vn, st, pos = oqk.qk_rows(rnd.streams, qkv_h, gq_h, gk_h, workloads.ROPE_THETA, workloads.NORM_EPS)
    gqf, gkf = obf16.to_f64(gq_h), obf16.to_f64(gk_h)
    exact_q, exact_k = [], []
    for r in range(rnd.R):
        row = obf16.to_f64(qkv_h[r])
        exact_q.append(_check_heads(Qg[r], row[:2048].reshape(32, 64), gqf, pos[r], f"q row {r}"))
        exact_k.append(_check_heads(K1[st[r]][:, pos[r]], row[2048:2560].reshape(8, 64), gkf, pos[r],
                                    f"k row {r}"))
        assert np.array_equal(V1[st[r]][:, pos[r]], Vn[r]), f"v row {r}"
    print(f"  exact-rounding share: q {np.mean(exact_q):.5f}, k {np.mean(exact_k):.5f}", flush=True)
    assert np.mean(exact_q) > 0.99 and np.mean(exact_k) > 0.99
    for s, (w, keys, _cap) in enumerate(rnd.streams):
        keep = np.ones(K0[s].shape[1], dtype=bool)
        keep[keys - w:keys] = False
        assert np.array_equal(K1[s][:, keep], K0[s][:, keep]), f"K outside the window, stream {s}"
        assert np.array_equal(V1[s][:, keep], V0[s][:, keep]), f"V outside the window, stream {s}"


def test_qk_then_attention_reads_the_appended_keys():
    """The tiny round with the qk stage in front: attention over the caches
    the qk stage just wrote matches the oracle's attention over the oracle's
    appended caches (the qk outputs taken from the GPU, so the check is the
    placement, not the rounding)."""
    from oracle import attn as oattn
    from oracle import table as otable
    rnd = workloads.Round(0, device="cuda", n_conv=0, n_attn=1, with_logits=False)
    qkv, gq, gk = workloads.qk_inputs(rnd.R, seed=77, device="cuda")
    K, V = rnd.attn[0][1], rnd.attn[0][2]
    rb = asv.RoundBuffers(rnd.streams, [], [K], [V], device="cuda")
    rb.upload()
    rb.qk(0, qkv, gq, gk, workloads.ROPE_THETA, workloads.NORM_EPS)
    rb.attn(0, rb.q)
    rb.merge()
    torch.cuda.synchronize()
    o = obf16.to_f64(_u16(rb.o))
    t = otable.build(rnd.streams)
    ref = oattn.attention(t, _u16(rb.q), [_u16(k) for k in K], [_u16(workloads.v_logical(v)) for v in V])
    assert np.abs(o - ref).max() <= 2e-2


@pytest.mark.parametrize("streams", [
    [(16, 16, 32), (1, 1, 32), (3, 131072, 131072)],   # window = cache (positions from 0), one key, the last position
    [(7, 40, 64)] * 5 + [(16, 4096, 4096)],
])
def test_qk_edge_streams(streams):
    print(f"qk edge: {streams}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    K, V = [], []
    for (_, keys, cap) in streams:
        k, v = workloads.kv_cache(keys, cap, g, "cuda")
        K.append(k)
        V.append(v)
    R = sum(w for w, _, _ in streams)
    qkv, gq, gk = workloads.qk_inputs(R, seed=5, device="cuda")
    K0 = [_u16(k) for k in K]
    V0 = [_u16(workloads.v_logical(v)) for v in V]
    rb = asv.RoundBuffers(streams, [], [K], [V], device="cuda")
    rb.upload()
    rb.qk(0, qkv, gq, gk, workloads.ROPE_THETA, workloads.NORM_EPS)
    torch.cuda.synchronize()
    Qg = _u16(rb.q)
    K1 = [_u16(k) for k in K]
    V1 = [_u16(workloads.v_logical(v)) for v in V]
    qkv_h = _u16(qkv)
    _, _, Vn, st, pos = oqk.qk_rows(streams, qkv_h, _u16(gq), _u16(gk), workloads.ROPE_THETA, workloads.NORM_EPS)
    gqf, gkf = obf16.to_f64(_u16(gq)), obf16.to_f64(_u16(gk))
    for r in range(R):
        row = obf16.to_f64(qkv_h[r])
        _check_heads(Qg[r], row[:2048].reshape(32, 64), gqf, pos[r], f"q row {r}")
        _check_heads(K1[st[r]][:, pos[r]], row[2048:2560].reshape(8, 64), gkf, pos[r], f"k row {r}")
        assert np.array_equal(V1[st[r]][:, pos[r]], Vn[r])
    for s, (w, keys, _cap) in enumerate(streams):
        keep = np.ones(K0[s].shape[1], dtype=bool)
        keep[keys - w:keys] = False
        assert np.array_equal(K1[s][:, keep], K0[s][:, keep]) and np.array_equal(V1[s][:, keep], V0[s][:, keep])
    assert pos.max() == max(k - 1 for _, k, _ in streams)
