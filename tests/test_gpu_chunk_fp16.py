"""The fp16 P.V path of prompt-chunk (group) items, against the oracle and
against exact scale invariance.

A group item rewrites each 32-key V quarter (one 16-wide d tile) in LDS as
fp16 scaled by 2^e, where e is a per-d-tile exponent that follows the
quarters' largest magnitudes (down at once when a quarter does not fit below
2^16, up when a quarter is far below what e allows), and rounds the weights
to fp16. These tests aim at what that design could get wrong:
- V of any magnitude: scaling V by 2^s must scale every partial o and every
  merged output by exactly 2^s and leave m and l bit-identical (the kernel's
  scale moves by exactly -s, so the fp16 operands are the same bits);
- weights in fp16's subnormal range (below 2^-14 of the base) must still
  count, in l and in o;
- d tiles of very different magnitudes, a scale that falls in the middle of
  an item, and whole zero sub-blocks at the start of an item: each d tile
  must stay within 1e-3 of its own largest |o|;
- a huge V value at a key of negligible weight: the scale must come back up
  after its sub-block.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import attn as oattn
from oracle import table as otable

from helpers import (bf16_to_f64, check_attention_layer, host_u16, oracle_attn_inputs,
                     run_round)

pytestmark = pytest.mark.gpu

# chunk streams of 6 and 3 tiles (group items of 4 + 2 and 3 tiles), a
# 5-row window and a one-row stream, so both item kinds run side by side
STREAMS = [(96, 3000, 3008), (40, 700, 704), (5, 900, 928), (1, 64, 64)]


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    import attention_stream_verify_amd as asv
    asv.lib()
    torch.cuda.init()


def _partials(rb, out):
    P = int(rb.info.partial_count)
    p = out["partials"][0]
    return p[:P * 64].view(P, 64).cpu().numpy(), p[P * 64:].view(P, 2).cpu().numpy()


def _scale_bf16_(t, s):
    """t (int16 view of bf16) *= 2^s in place; exact inside bf16's range."""
    t.copy_((t.view(torch.bfloat16).float() * 2.0 ** s).to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("s", [-80, -40, 40, 100])
def test_v_scale_invariance_bitwise(s):
    print(f"\n[fp16] V scaled by 2^{s}: {STREAMS}", flush=True)
    rnd = workloads.Round(0, "cuda", n_conv=0, n_attn=1, streams=STREAMS, with_logits=False)
    rb0, out0 = run_round(rnd, with_argmax=False)
    o0, ml0 = _partials(rb0, out0)
    m0 = bf16_to_f64(host_u16(out0["o"][0]))
    for v in rnd.attn[0][2]:
        _scale_bf16_(v, s)
    rb1, out1 = run_round(rnd, with_argmax=False)
    o1, ml1 = _partials(rb1, out1)
    m1 = bf16_to_f64(host_u16(out1["o"][0]))
    assert np.array_equal(ml0, ml1), "m, l must not depend on V"
    assert np.isfinite(o0).all() and np.isfinite(o1).all()
    assert np.array_equal(o1, np.ldexp(o0, s).astype(np.float32)), \
        f"partials not scaled exactly: max |d| {np.abs(o1 - np.ldexp(o0, s)).max():.3e}"
    assert np.array_equal(m1, np.ldexp(m0, s)), "merged outputs not scaled exactly"


def test_weights_below_fp16_normal_range():
    """One key at weight 1 and ~3,000 at exp(-11) ~ 2^-15.9 (fp16
    subnormals): they carry ~5% of l, which a flush to zero would lose."""
    streams = [(64, 3000, 3008)]
    print(f"\n[fp16] weights in the fp16 subnormal range: {streams}", flush=True)
    rnd = workloads.Round(0, "cuda", n_conv=0, n_attn=1, streams=streams, with_logits=False)
    Q, ks, _ = rnd.attn[0]
    q = torch.zeros(Q.shape, dtype=torch.float32, device=Q.device)
    q[..., 0] = 16.0
    Q.copy_(q.to(torch.bfloat16).view(torch.int16))
    k = torch.zeros((ks[0].shape[0], 3000, ks[0].shape[2]), dtype=torch.float32, device=Q.device)
    k[:, 0, 0] = 8.0      # score 128 x 1/8: weight 1 at the base
    k[:, 1:, 0] = 2.5     # score 40 x 1/8: weight exp(-11)
    ks[0][:, :3000].copy_(k.to(torch.bfloat16).view(torch.int16))
    rb, out = run_round(rnd, with_argmax=False)
    t = otable.build(streams)
    rows = list(range(t.n_rows))
    prel, oerr = check_attention_layer(rnd, rb, out["partials"][0], out["o"][0], 0, rows,
                                       "fp16-subnormal weights")
    print(f"[fp16] subnormal weights: partial o rel err {prel:.2e}, output abs err {oerr:.2e}",
          flush=True)
    # the small weights' share of l is large enough that losing them fails
    _, _, ref_l, _ = oattn.partials(t, *oracle_attn_inputs(rnd, 0), rows=[0])
    assert ref_l[t.record(0, 0, 0)] > 1.04


def _check_per_d_tile(got, ref, bound, what):
    """|got - ref| <= bound x (largest |ref| of the same record and d tile)."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, 4, 16)
    r = np.asarray(ref, dtype=np.float64).reshape(-1, 4, 16)
    scale = np.abs(r).max(axis=2, keepdims=True)
    err = np.abs(g - r)
    bad = err > bound * scale
    assert not bad.any(), f"{what}: {int(bad.sum())} outside, max rel " \
        f"{float((err / np.where(scale > 0, scale, 1)).max()):.3e}"
    return float((err / np.where(scale > 0, scale, 1)).max())


def test_v_scales_per_d_tile():
    streams = [(96, 3000, 3008), (48, 1200, 1216)]
    print(f"\n[fp16] per-d-tile V scales: {streams}", flush=True)
    rnd = workloads.Round(0, "cuda", n_conv=0, n_attn=1, streams=streams, with_logits=False)
    vs = rnd.attn[0][2]
    v0 = workloads.v_logical(vs[0]).view(torch.bfloat16).float()
    keys0 = streams[0][1]
    v0[:, :keys0, 16:32] *= 2.0 ** 30     # d tile 1 large
    v0[:, :keys0, 32:48] *= 2.0 ** -30    # d tile 2 small
    v0[:, :1000, 48:64] *= 2.0 ** -10     # d tile 3 grows at key 1,000: its scale falls
    v0[:, 1500, 5] = 2.0 ** 20            # one large value in the middle of d tile 0
    vs[0].copy_(workloads.v_blocked(v0.to(torch.bfloat16).view(torch.int16)))
    v1 = workloads.v_logical(vs[1]).view(torch.bfloat16).float()
    v1[:, :64, :] = 0.0                   # the first two sub-blocks all zero
    vs[1].copy_(workloads.v_blocked(v1.to(torch.bfloat16).view(torch.int16)))

    rb, out = run_round(rnd, with_argmax=False)
    t = otable.build(streams)
    rows = list(range(t.n_rows))
    Qh, Kh, Vh = oracle_attn_inputs(rnd, 0)
    ref_o, ref_m, ref_l, _ = oattn.partials(t, Qh, Kh, Vh, rows=rows)
    dense = oattn.attention(t, Qh, Kh, Vh, rows=rows)
    po, pml = _partials(rb, out)
    recs = [t.record(r, h, sp) for r in rows for h in range(32) for sp in range(t.row_nsplit(r))]
    recs = np.asarray(recs, dtype=np.int64)
    assert np.all(np.abs(pml[recs, 0] - ref_m[recs]) <= 1e-3 * np.maximum(1.0, np.abs(ref_m[recs])))
    assert np.all(np.abs(pml[recs, 1] - ref_l[recs]) <= 1e-3 * ref_l[recs])
    prel = _check_per_d_tile(po[recs], ref_o[recs], 1e-3, "partials")
    # merged bf16 output: half a bf16 step of the tile's largest value, plus
    # the partials' bound
    g = bf16_to_f64(host_u16(out["o"][0]))[rows]
    orel = _check_per_d_tile(g.reshape(-1, 64), dense[rows].reshape(-1, 64), 2.0 ** -8 + 1e-3,
                             "merged output")
    print(f"[fp16] per-d-tile scales: partial rel err {prel:.2e}, output rel err {orel:.2e}",
          flush=True)


def test_v_outlier_with_negligible_weight():
    """One V value 2^30 (d tile 0) at a key whose weight is about e^-40:
    its sub-block's quarter takes a scale 2^-30 lower, and the next quarters
    must take the scale back up, or every later value of that d tile would
    keep only a few bits."""
    streams = [(64, 3000, 3008)]
    print(f"\n[fp16] V outlier at a negligible weight: {streams}", flush=True)
    rnd = workloads.Round(0, "cuda", n_conv=0, n_attn=1, streams=streams, with_logits=False)
    Q, ks, vs = rnd.attn[0]
    q = Q.view(torch.bfloat16).float()
    q[..., 0] = 4.0           # with k[100][0] = -80: 40 off every score of key 100
    Q.copy_(q.to(torch.bfloat16).view(torch.int16))
    k = ks[0].view(torch.bfloat16).float()
    k[:, 100, 0] = -80.0
    ks[0].copy_(k.to(torch.bfloat16).view(torch.int16))
    v = workloads.v_logical(vs[0]).view(torch.bfloat16).float()
    v[:, 100, 0:16] = 2.0 ** 30
    vs[0].copy_(workloads.v_blocked(v.to(torch.bfloat16).view(torch.int16)))

    rb, out = run_round(rnd, with_argmax=False)
    t = otable.build(streams)
    rows = list(range(t.n_rows))
    Qh, Kh, Vh = oracle_attn_inputs(rnd, 0)
    ref_o, ref_m, ref_l, _ = oattn.partials(t, Qh, Kh, Vh, rows=rows)
    dense = oattn.attention(t, Qh, Kh, Vh, rows=rows)
    po, pml = _partials(rb, out)
    recs = [t.record(r, h, sp) for r in rows for h in range(32) for sp in range(t.row_nsplit(r))]
    recs = np.asarray(recs, dtype=np.int64)
    # the outlier must not dominate: the reference's d tile 0 stays small
    assert np.abs(ref_o[recs, :16]).max() < 16.0
    assert np.all(np.abs(pml[recs, 1] - ref_l[recs]) <= 1e-3 * ref_l[recs])
    prel = _check_per_d_tile(po[recs], ref_o[recs], 1e-3, "partials")
    g = bf16_to_f64(host_u16(out["o"][0]))[rows]
    orel = _check_per_d_tile(g.reshape(-1, 64), dense[rows].reshape(-1, 64), 2.0 ** -8 + 1e-3,
                             "merged output")
    print(f"[fp16] V outlier: partial rel err {prel:.2e}, output rel err {orel:.2e}", flush=True)
