"""Planted cross-stream controls: the parity checks must go red when the
table sends every stream to the first stream's buffers.

PR #1377 "LFM2: shared-round decode", "Kernel contract and exactness": the
checks are only trusted if planted mistakes fail them, among them a round in
which all streams take their conv state from the first stream and one in
which all streams put their K/V into the first stream's cache.

The builder refuses a table whose streams share a buffer (ASV_E_ARG), so each
control builds a valid table, then rewrites the address arrays of the host
blob after the build and before the upload: every stream's entry is set to
stream 0's. The streams of each control have equal capacities (conv states
are all [2][2048]; K/V caches all hold 256 keys), so every redirected access
stays inside a live allocation of the size the kernel assumes. Each control
first runs unpatched and must pass, then patched and must fail: the check is
shown to be sensitive to exactly the planted mistake.
"""

import numpy as np
import pytest
import torch

import attention_stream_verify_amd as asv
import workloads
from oracle import conv as oconv
from oracle import qk as oqk
from oracle import table as otable

from helpers import check_attention_layer, check_bf16_out, host_u16, run_round

pytestmark = pytest.mark.gpu

# four streams of different windows and equal caches with every slot a key
EQUAL_STREAMS = [(1, 256, 256), (2, 256, 256), (3, 256, 256), (4, 256, 256)]


def _point_every_stream_at_stream0(rb, field):
    """Rewrite the blob's per-layer address array `field` ('conv', 'k' or
    'v') so that every stream's entry is stream 0's, then upload."""
    info = rb.info
    S = int(info.n_streams)
    off = {"conv": info.off_conv_state, "k": info.off_k, "v": info.off_v}[field]
    n_layers = int(info.n_conv_layers if field == "conv" else info.n_attn_layers)
    arr = rb.blob_host[int(off): int(off) + 8 * n_layers * S].view(torch.int64).view(n_layers, S)
    first = arr[:, :1].clone()
    arr[:, :] = first
    assert len(set(arr.flatten().tolist())) == n_layers
    rb.upload()


def _conv_check(rnd, y, states, before):
    t = otable.build(rnd.streams)
    X, W, _ = rnd.conv[0]
    y_ref, st_ref = oconv.shared_conv(t, host_u16(X), host_u16(W), before)
    check_bf16_out(host_u16(y), y_ref, "conv output")
    for s, st in enumerate(states):
        assert np.array_equal(host_u16(st), st_ref[s]), f"state of stream {s}"


def test_control_every_stream_reads_stream0_conv_state():
    print("\n[control] conv state of stream 0 for every stream", flush=True)
    rnd = workloads.Round(0, "cuda", n_conv=1, n_attn=0, with_logits=False)
    X, W, states = rnd.conv[0]
    st0 = [s.clone() for s in states]
    before = [host_u16(s) for s in states]
    rb = asv.RoundBuffers(rnd.streams, [states], [], [])
    rb.upload()
    rb.conv(0, X, W)
    torch.cuda.synchronize()
    _conv_check(rnd, rb.y, states, before)                   # unpatched: green
    for s, st in zip(states, st0):
        s.copy_(st)
    _point_every_stream_at_stream0(rb, "conv")
    rb.conv(0, X, W)
    torch.cuda.synchronize()
    with pytest.raises(AssertionError):
        _conv_check(rnd, rb.y, states, before)               # planted: red


# a prompt chunk (40 rows: one group item of three tiles a head and split)
# and a 17-row stream (a group of two tiles) beside a window, caches alike
EQUAL_STREAMS_CHUNKS = [(40, 256, 256), (2, 256, 256), (17, 256, 256)]


@pytest.mark.parametrize("streams", [EQUAL_STREAMS, EQUAL_STREAMS_CHUNKS], ids=["windows", "chunks"])
def test_control_every_stream_reads_stream0_kv_cache(streams):
    print(f"\n[control] K/V cache of stream 0 read by every stream {streams}", flush=True)
    for field in ("k", "v"):
        rnd = workloads.Round(0, "cuda", n_conv=0, n_attn=1, streams=streams,
                              with_logits=False)
        rb, out = run_round(rnd, with_argmax=False)
        rows = list(range(rnd.R))
        check_attention_layer(rnd, rb, out["partials"][0], out["o"][0], 0, rows, "unpatched")
        _point_every_stream_at_stream0(rb, field)
        rb.attn(0, rnd.attn[0][0])
        rb.merge()
        torch.cuda.synchronize()
        print(f"[control] {field} redirected", flush=True)
        with pytest.raises(AssertionError):
            check_attention_layer(rnd, rb, rb.partials, rb.o, 0, rows, f"planted {field}")


def _qk_cache_check(streams, qkv, gq, gk, K, V, K0, V0):
    """Every stream's window keys and values at their positions of its own
    cache, and every other cache entry unchanged."""
    K1 = [host_u16(k) for k in K]
    V1 = [host_u16(workloads.v_logical(v)) for v in V]
    _, Kn, Vn, st, pos = oqk.qk_rows(streams, host_u16(qkv), host_u16(gq), host_u16(gk),
                                     workloads.ROPE_THETA, workloads.NORM_EPS)
    for r in range(len(st)):
        assert np.array_equal(V1[st[r]][:, pos[r]], Vn[r]), f"v row {r}"
        # k is rounded once by both sides from the same float64 value in all
        # but a few ulp cases; one bf16 step is the bound
        got = (K1[st[r]][:, pos[r]].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ref = (Kn[r].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
        assert np.all(np.abs(got - ref) <= step), f"k row {r}"
    for s, (w, keys, _cap) in enumerate(streams):
        keep = np.ones(K0[s].shape[1], dtype=bool)
        keep[keys - w:keys] = False
        assert np.array_equal(K1[s][:, keep], K0[s][:, keep]), f"K outside the window, stream {s}"
        assert np.array_equal(V1[s][:, keep], V0[s][:, keep]), f"V outside the window, stream {s}"


def test_control_every_stream_writes_stream0_cache():
    print("\n[control] qk stage writing every stream's K/V into stream 0's cache", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    K, V = [], []
    for (_, keys, cap) in EQUAL_STREAMS:
        k, v = workloads.kv_cache(keys, cap, g, "cuda")
        K.append(k)
        V.append(v)
    Kd0, Vd0 = [k.clone() for k in K], [v.clone() for v in V]
    K0 = [host_u16(k) for k in K]
    V0 = [host_u16(workloads.v_logical(v)) for v in V]
    R = sum(w for w, _, _ in EQUAL_STREAMS)
    qkv, gq, gk = workloads.qk_inputs(R, seed=9, device="cuda")
    rb = asv.RoundBuffers(EQUAL_STREAMS, [], [K], [V], device="cuda")
    rb.upload()
    rb.qk(0, qkv, gq, gk, workloads.ROPE_THETA, workloads.NORM_EPS)
    torch.cuda.synchronize()
    _qk_cache_check(EQUAL_STREAMS, qkv, gq, gk, K, V, K0, V0)   # unpatched: green
    for t, t0 in zip(K + V, Kd0 + Vd0):
        t.copy_(t0)
    _point_every_stream_at_stream0(rb, "k")
    _point_every_stream_at_stream0(rb, "v")
    rb.qk(0, qkv, gq, gk, workloads.ROPE_THETA, workloads.NORM_EPS)
    torch.cuda.synchronize()
    with pytest.raises(AssertionError):
        _qk_cache_check(EQUAL_STREAMS, qkv, gq, gk, K, V, K0, V0)  # planted: red
