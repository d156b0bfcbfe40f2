"""Shared helpers of the GPU parity tests: device rounds, host copies, and the
comparison rules (tolerances written out here, used by every parity test)."""

import numpy as np
import torch

import workloads
from oracle import attn as oattn
from oracle import table as otable


def host_u16(t):
    return t.detach().cpu().numpy().view(np.uint16)


def bf16_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------- compare rules

def check_bf16_out(gpu_bits, ref64, what):
    """|gpu - ref| <= max(2e-2, 2^-8 |ref|): the bf16-output bound.

    2e-2 absolute is the bound for attention and conv outputs; above
    |ref| = 5.12 half a bf16 step exceeds it, so the bound widens to 2^-8 |ref|
    (half a step), the best any correctly rounded bf16 value can do.
    """
    g = bf16_to_f64(gpu_bits)
    ref = np.asarray(ref64, dtype=np.float64)
    assert np.isfinite(g).all(), f"{what}: nonfinite output"
    err = np.abs(g - ref)
    bound = np.maximum(2e-2, np.abs(ref) * 2.0 ** -8)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside the bound, "
                           f"max err {err.max():.3e}")
    return float(err.max())


def check_partials(po, pml, ref_o, ref_m, ref_l, recs, what):
    """fp32 partials within 1e-3 relative: m to 1e-3 max(1,|m|), l to 1e-3 l,
    o to 1e-3 of the record's largest |o| (element-relative is ill-posed for
    entries near zero)."""
    recs = np.asarray(recs, dtype=np.int64)
    gm, gl, go = pml[recs, 0].astype(np.float64), pml[recs, 1].astype(np.float64), po[recs].astype(np.float64)
    rm, rl, ro = ref_m[recs], ref_l[recs], ref_o[recs]
    assert np.all(np.abs(gm - rm) <= 1e-3 * np.maximum(1.0, np.abs(rm))), f"{what}: m"
    assert np.all(np.abs(gl - rl) <= 1e-3 * rl), f"{what}: l"
    scale = np.abs(ro).max(axis=1, keepdims=True)
    err = np.abs(go - ro)
    assert np.all(err <= 1e-3 * scale), f"{what}: o max rel {float((err / scale).max()):.3e}"
    return float((err / scale).max())


# ----------------------------------------------------------- device rounds

def run_round(rnd, layers_conv=None, layers_attn=None, with_argmax=True, full=False):
    """Run a workloads.Round through the library on the current device
    (full: with a block attention table).

    Returns the RoundBuffers and, per layer, the outputs (cloned)."""
    import attention_stream_verify_amd as asv
    convs = [[st for st in layer[2]] for layer in rnd.conv]
    ks = [layer[1] for layer in rnd.attn]
    vs = [layer[2] for layer in rnd.attn]
    vocab = rnd.logits.shape[1] if (with_argmax and rnd.logits is not None) else None
    rb = asv.RoundBuffers(rnd.streams, convs, ks, vs, device=rnd.attn[0][0].device if rnd.attn else "cuda",
                          vocab=vocab, full=full)
    rb.upload()
    out = {"y": [], "o": [], "partials": [], "states": []}
    for li in (range(rnd.n_conv) if layers_conv is None else layers_conv):
        X, W, _ = rnd.conv[li]
        rb.conv(li, X, W)
        out["y"].append(rb.y.clone())
    for li in (range(rnd.n_attn) if layers_attn is None else layers_attn):
        Q = rnd.attn[li][0]
        rb.attn(li, Q)
        rb.merge()
        out["partials"].append(rb.partials.clone())
        out["o"].append(rb.o.clone())
    if vocab is not None:
        rb.argmax(rnd.logits)
        out["pick"] = rb.pick.clone()
        out["flag"] = rb.flag.clone()
    torch.cuda.synchronize()
    return rb, out


def oracle_attn_inputs(rnd, li):
    Q, ks, vs = rnd.attn[li]
    Qh = host_u16(Q)
    Kh = [host_u16(k) for k in ks]
    Vh = [host_u16(workloads.v_logical(v)) for v in vs]
    return Qh, Kh, Vh


def sample_rows(table, n_extra, seed):
    """First and last row of every stream, plus n_extra seeded random rows."""
    rows = set()
    for s in range(len(table.rows)):
        rows.add(int(table.seg_off[s]))
        rows.add(int(table.seg_off[s + 1]) - 1)
    rng = np.random.default_rng(seed)
    for r in rng.integers(0, table.n_rows, size=n_extra):
        rows.add(int(r))
    return sorted(rows)


def sample_rows_every_tile(table, n_extra, seed):
    """Rows from every segment and every tile: the first, a middle and the
    last row of each stream; for streams longer than one tile (prompt chunks)
    the first row of every 16-row tile (the row that sees the fewest of the
    tile's keys, where the causal mask cuts deepest into the tile's last
    sub-blocks) and the last row of every fourth tile; plus n_extra seeded
    random rows."""
    rows = set()
    for s in range(len(table.rows)):
        a, b = int(table.seg_off[s]), int(table.seg_off[s + 1])
        rows.update((a, (a + b - 1) // 2, b - 1))
    for (s, row0, nrows, pos0) in table.tiles:
        if table.rows[int(s)] > otable.TILE_ROWS:
            rows.add(int(row0))
            if (int(pos0) // otable.TILE_ROWS) % 4 == 3:
                rows.add(int(row0) + int(nrows) - 1)
    rng = np.random.default_rng(seed)
    for r in rng.integers(0, table.n_rows, size=n_extra):
        rows.add(int(r))
    return sorted(rows)


def chunk_rows(table, rows):
    """The rows of `rows` that belong to streams longer than one tile."""
    return [r for r in rows if table.rows[int(table.row_stream[r])] > otable.TILE_ROWS]


def check_attention_layer(rnd, rb, partials, o_bits, li, rows, what, full=False):
    """Compare a layer's partials (every record of `rows`) and merged output."""
    t = otable.build(rnd.streams, full=full)
    Qh, Kh, Vh = oattn_inputs = oracle_attn_inputs(rnd, li)
    del oattn_inputs
    ref_o, ref_m, ref_l, _ = oattn.partials(t, Qh, Kh, Vh, rows=rows)
    dense = oattn.attention(t, Qh, Kh, Vh, rows=rows)
    P = int(rb.info.partial_count)
    po = partials[:P * 64].view(P, 64).cpu().numpy()
    pml = partials[P * 64:].view(P, 2).cpu().numpy()
    recs = []
    for r in rows:
        for h in range(32):
            for sp in range(t.row_nsplit(r)):
                recs.append(t.record(r, h, sp))
    prel = check_partials(po, pml, ref_o, ref_m, ref_l, recs, what + " partials")
    # empty records a tile wrote for its shorter rows: exactly (-inf, 0, 0)
    for r in rows:
        s = int(t.row_stream[r])
        tile = [tt for tt in t.tiles if tt[1] <= r < tt[1] + tt[2]][0]
        last = t.keys[s] if full else t.keys[s] - t.rows[s] + tile[3] + tile[2]
        for sp in range(t.row_nsplit(r), t.splits_before(s, last)):
            for h in range(32):
                rec = t.record(r, h, sp)
                assert pml[rec, 0] == -np.inf and pml[rec, 1] == 0 and not po[rec].any(), what
    oerr = check_bf16_out(host_u16(o_bits)[rows], dense[rows], what + " output")
    return prel, oerr
