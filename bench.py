"""Benchmark of one shared verify round on one MI355X.

A step is one whole round over a synthetic workload already resident in HBM:
the table upload, 30 gated short-conv layers, 10 attention layers (split-K
attention + merge) and the argmax over 128,000-wide logits, every layer on
its own buffers. Default workload: long context, 4 streams x 16 window rows
(64 rows) with 65,536 / 98,304 / 130,816 / 131,072 keys.

Prints one JSON line: verify rows/s per round (and the round time's median,
p10 and p90); the roofline of the attention kernel (algorithmic K/V + Q bytes
per launch over its average launch time, timed with HIP events on the stream
it runs on, against 8 TB/s); attention + merge per layer (K/V + Q + O bytes
over the pair's time; alternate rounds time the pair with no event between
the two kernels and the attention alone); the profiled HBM traffic and MFMA
busy fraction when profiles/ holds them for these kernel sources; the host
table build time; the CPU oracle timed on a bounded sample of the same
workload; and a per-workload object: every workload (tiny, 16 x 1 decode,
16 x 8 verify, 4 x 16 long context, the 2,048-row scratch) measured in the
same run the same way -- rows/s, round time, the attention launch against
8 TB/s and against its max(bytes / 8 TB/s, flops / 2.5 PFLOP/s) bound, and
the attention + merge pair.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak
WORKLOAD_NAMES = {
    0: "tiny: 4 streams, windows 1-4, keys 16-256",
    1: "decode: 16 streams x 1 row, keys 512-4096",
    2: "draft verify: 16 streams x 8 rows, keys 2k-32k",
    3: "long context: 4 streams x 16 rows, keys 65,536-131,072",
    4: "full scratch: 2,048 rows, 48 windows + prompt chunks, lognormal keys",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=3, choices=[0, 1, 2, 3, 4])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-markov", action="store_true", help="skip the Markov-head timing leg")
    p.add_argument("--no-workloads", action="store_true",
                   help="skip the per-workload object (every workload's round, measured in this run)")
    p.add_argument("--workload-steps", type=int, default=10,
                   help="timed rounds of each workload of the per-workload object")
    p.add_argument("--eager", action="store_true",
                   help="time the rounds as eager launches (default: replays of one captured HIP graph)")
    p.add_argument("--with-qk", action="store_true",
                   help="run the qk stage before every attention layer inside the timed round")
    p.add_argument("--block", action="store_true",
                   help="attention through a block table: every row sees all of its stream's keys")
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB three times (the known-size "
                        "kernel that scales HBM byte counters) and exit")
    return p.parse_args()


def calibrate_copy(mib):
    """A plain copy of a known size: its FETCH_SIZE / WRITE_SIZE counters give
    the factor between those counters and the bytes a kernel really moves."""
    import torch
    n = mib << 20
    src = torch.randint(0, 127, (n,), dtype=torch.int8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "reads": n, "writes": n}), flush=True)


WORKLOAD_KEYS = {0: "tiny", 1: "decode_16x1", 2: "verify_16x8", 3: "long_context_4x16",
                 4: "scratch_2048"}


TRAFFIC_PROFILES = {3: "profiles/attn_split_long_context_traffic.md",
                    4: "profiles/attn_split_scratch_traffic.md"}


def profiled_traffic(config):
    """HBM bytes a launch of the attention kernel moved under rocprofv3
    (FETCH_SIZE and WRITE_SIZE passes, scaled by a plain-copy calibration),
    as recorded in profiles/ -- or None when there is no profile for this
    workload or the kernel sources changed since it was taken."""
    f = profile_fields(TRAFFIC_PROFILES.get(config), ("traffic_bytes_per_launch",))
    return None if f is None else int(f["traffic_bytes_per_launch"])


SQ_PROFILES = {1: "profiles/attn_split_decode_sq_counters.md",
               2: "profiles/attn_split_verify_sq_counters.md",
               3: "profiles/attn_split_long_context_sq_counters.md",
               4: "profiles/attn_split_scratch_sq_counters.md"}


def profile_fields(name, keys):
    """Fields of a profile summary in profiles/, or None when it is missing or
    the kernel sources changed since it was taken (their sha256 is recorded)."""
    import hashlib
    if name is None or not os.path.exists(os.path.join(ROOT, name)):
        return None
    fields = {}
    for line in open(os.path.join(ROOT, name)):
        if ":" in line and line.split(":", 1)[0].strip() in keys + ("kernel_sources_sha256",
                                                                   "kernel_sources"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if "kernel_sources" not in fields or "kernel_sources_sha256" not in fields:
        return None
    h = hashlib.sha256()
    for src in fields["kernel_sources"].split():
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != fields["kernel_sources_sha256"] or any(k not in fields for k in keys):
        return None
    return fields


def profiled_mfma(config):
    """MFMA pipe busy fraction of the attention kernel from SQ counters
    (SQ_VALU_MFMA_BUSY_CYCLES over SIMD cycles), as recorded in profiles/."""
    f = profile_fields(SQ_PROFILES.get(config), ("mfma_busy_frac", "valu_active_frac"))
    if f is None:
        return None
    return {"mfma_busy_frac": float(f["mfma_busy_frac"]), "valu_active_frac": float(f["valu_active_frac"]),
            "source": SQ_PROFILES[config]}


def layer_order(n_conv, n_attn):
    """Interleave the layers as the model does: every fourth layer attends."""
    order, c, a = [], 0, 0
    while c < n_conv or a < n_attn:
        if a < n_attn and (len(order) % 4 == 3 or c >= n_conv):
            order.append(("attn", a))
            a += 1
        else:
            order.append(("conv", c))
            c += 1
    return order


def cpu_baseline(rnd, R, full=False):
    """The oracle, as it stands, on one conv layer, one attention layer and the
    argmax of this workload, scaled to a round by 30 / 10 / 1."""
    import numpy as np

    import workloads
    from oracle import argmax as oargmax
    from oracle import attn as oattn
    from oracle import conv as oconv
    from oracle import table as otable

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1

    def u16(t):
        return t.detach().cpu().numpy().view(np.uint16)

    X, W, states = rnd.conv[0]
    Q, ks, vs = rnd.attn[0]
    Xh, Wh, sth = u16(X), u16(W), [u16(s) for s in states]
    Qh, Kh = u16(Q), [u16(k) for k in ks]
    Vh = [u16(workloads.v_logical(v)) for v in vs]
    Lh = u16(rnd.logits)
    t = otable.build(rnd.streams, full=full)
    t0 = time.perf_counter()
    oconv.shared_conv(t, Xh, Wh, sth)
    t1 = time.perf_counter()
    po, pm, pl, _ = oattn.partials(t, Qh, Kh, Vh)
    oattn.merge(t, po, pm, pl)
    t2 = time.perf_counter()
    oargmax.row_argmax(Lh)
    t3 = time.perf_counter()
    t_round = rnd.n_conv * (t1 - t0) + rnd.n_attn * (t2 - t1) + (t3 - t2)
    return {
        "value": R / t_round, "unit": "rows/s", "cores": int(cores), "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": (f"one conv layer ({t1 - t0:.2f} s), one attention layer with partials "
                   f"and merge ({t2 - t1:.2f} s) and the argmax ({t3 - t2:.2f} s) over all "
                   f"{R} rows of this workload, scaled by {rnd.n_conv}/{rnd.n_attn}/1 "
                   f"to a {t_round:.1f} s round"),
    }


def markov_leg(torch, asv, dev, seed, calls=20):
    """One Markov-head pass of the drafter: 4 chains x depth 8 (a hold pass
    holds at most 32 rows), vocabulary 128,000, rank 256, random bf16
    weights, in the form asv_markov_pick chooses (resident: W2 read once a
    pass and kept in registers) and, for comparison, one launch a depth (W2
    read once a depth). Bytes of the chosen form: W2 once, each chain's
    logit rows, the W1 rows (512 bytes each); its arithmetic: one float32
    fused multiply-add per token, rank index, chain and depth."""
    vocab, rank, chains = 128000, 256, [(0, 8), (8, 8), (16, 8), (24, 8)]
    rows, depth = 32, 8
    g = torch.Generator(device=dev)
    g.manual_seed(seed + 101)

    def bf16(shape, scale):
        x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32) * scale
        return x.to(torch.bfloat16).view(torch.int16)

    w1, w2, base = bf16((vocab, rank), 0.3), bf16((vocab, rank), 0.3), bf16((rows, vocab), 3.0)
    w2c = torch.empty_like(w2)
    asv.markov_pack_w2(w2, vocab, rank, w2c)
    prev0 = torch.tensor([17, 4242, 90000, 127999], dtype=torch.int32, device=dev)
    pick = torch.empty(rows, dtype=torch.int32, device=dev)
    flag = torch.empty(rows, dtype=torch.uint8, device=dev)
    ws = torch.empty(asv.markov_workspace(vocab), dtype=torch.uint8, device=dev)

    def timed(form):
        def call():
            asv.markov_pick(base, rows, vocab, chains, prev0, w1, w2c, vocab, rank, pick, flag, ws, form=form)
        for _ in range(3):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(calls):
            call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / calls

    us_launches = timed("launches")
    launches_bytes = depth * vocab * rank * 2 + rows * vocab * 2 + rows * rank * 2
    try:                             # the form asv_markov_pick takes when the device admits it
        us, form, n_launch = timed("resident"), "resident", 2
        nbytes = vocab * rank * 2 + rows * vocab * 2 + rows * rank * 2
    except asv.AsvError:
        us, form, n_launch, nbytes = us_launches, "launches", depth + 1, launches_bytes
    fmas = depth * vocab * rank * len(chains)
    fma_peak = 256 * 64 * 2.4e9      # non-packed float32 FMA lanes of 256 CUs at 2.4 GHz
    return {"shape": "4 chains x depth 8, vocab 128,000, rank 256", "form": form,
            # resident: W2 leaves HBM once a pass, and the pass is a chain of
            # depths (record exchange, W1 rows, scoring); one launch a depth
            # reads W2 at every depth and is bound by HBM
            "bound": "alu" if form == "resident" else "hbm",
            "avg_call_us": us, "launches_per_call": n_launch, "bytes_per_call": nbytes,
            "achieved_gbs": nbytes / (us * 1e-6) / 1e9,
            "frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "fmas_per_call": fmas, "fma_frac": fmas / (us * 1e-6) / fma_peak,
            "launches_form_avg_call_us": us_launches,
            "launches_form_bytes_per_call": launches_bytes,
            "launches_form_frac": launches_bytes / (us_launches * 1e-6) / 1e9 / HBM_PEAK_GBS}


def measure_round(torch, asv, workloads, dev, config, steps, warmup, block=False, with_qk=False,
                  eager=False, seed=None):
    """Build one workload's inputs and time its rounds.

    Eager rounds (events on torch's current stream, the stream the library
    launches on) give the per-kernel times: odd rounds record events around
    each attention launch alone, even rounds around each attention + merge
    pair (no event between the two kernels). Then, unless eager, the round is
    captured once as a HIP graph (the table upload and every launch) and
    replayed: ``ms_step`` is the replays' time per round, the same work with
    the host's per-launch cost taken out. Returns the measurements and the
    objects the other legs reuse."""
    rnd = workloads.Round(config, device=dev, seed=seed)
    R, S = rnd.R, rnd.S
    rb = asv.RoundBuffers(rnd.streams, [layer[2] for layer in rnd.conv],
                          [layer[1] for layer in rnd.attn], [layer[2] for layer in rnd.attn],
                          device=dev, vocab=rnd.logits.shape[1], full=block)
    order = layer_order(rnd.n_conv, rnd.n_attn)
    sum_keys = sum(k for _, k, _ in rnd.streams)
    attn_bytes = 2048 * sum_keys + 4096 * R            # K/V once + Q, per launch
    # algorithmic attention flops a launch: q.k and p.v, 2 * 64 multiply-adds
    # each, for every (row, q head, visible key)
    visible = sum((k if block else k - w + i + 1) for w, k, _ in rnd.streams for i in range(w))
    attn_flops = 4 * 64 * 32 * visible
    merge_bytes = 4096 * R                              # O written (partials are a means)
    qkv, gq, gk = workloads.qk_inputs(R, seed=rnd.seed + 7, device=dev)

    def event():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def step(ev=None, split=False):
        """One round; with ev, events: round start, per attention layer
        (start, end of the attention alone when split, else of the pair),
        round end."""
        if ev is not None:
            ev.append([event()])
        rb.upload()
        for kind, i in order:
            if kind == "conv":
                X, W, _ = rnd.conv[i]
                rb.conv(i, X, W)
            else:
                if with_qk:
                    rb.qk(i, qkv, gq, gk, workloads.ROPE_THETA, workloads.NORM_EPS)
                if ev is not None:
                    ev[-1].append(event())
                rb.attn(i, rb.q if with_qk else rnd.attn[i][0])
                if ev is not None and split:
                    ev[-1].append(event())
                rb.merge()
                if ev is not None and not split:
                    ev[-1].append(event())
        rb.argmax(rnd.logits)
        if ev is not None:
            ev[-1].append(event())

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = []
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(steps):
        step(ev, split=(k % 2 == 1))
    stop.record()
    torch.cuda.synchronize()
    eager_ms_step = start.elapsed_time(stop) / steps
    round_ms = sorted(e[0].elapsed_time(e[-1]) for e in ev)
    attn_ms, pair_ms = [], []
    for k, e in enumerate(ev):
        for j in range(1, len(e) - 1, 2):
            (attn_ms if k % 2 == 1 else pair_ms).append(e[j].elapsed_time(e[j + 1]))
    if not attn_ms:  # a single timed round: time attention alone in it
        attn_ms = pair_ms
    ms_step = eager_ms_step
    if not eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        ms_step = g0.elapsed_time(g1) / steps
        del graph
        # the attention launches alone, every layer in one captured graph and
        # replayed: kernel time without the host's per-launch latency, which
        # the eager events above include for short launches
        agraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(agraph):
            for i in range(rnd.n_attn):
                rb.attn(i, rb.q if with_qk else rnd.attn[i][0])
        for _ in range(warmup):
            agraph.replay()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(steps):
            agraph.replay()
        a1.record()
        torch.cuda.synchronize()
        attn_graph_us = a0.elapsed_time(a1) / (steps * rnd.n_attn) * 1e3
        del agraph
    else:
        attn_graph_us = None
    return {
        "rnd": rnd, "rb": rb, "R": R, "S": S, "sum_keys": sum_keys, "attn_bytes": attn_bytes,
        "attn_flops": attn_flops, "merge_bytes": merge_bytes, "qkv": (qkv, gq, gk),
        "ms_step": ms_step, "eager_ms_step": eager_ms_step, "round_ms": round_ms,
        "attn_us": sum(attn_ms) / len(attn_ms) * 1e3, "pair_us": sum(pair_ms) / len(pair_ms) * 1e3,
        "attn_graph_us": attn_graph_us,
    }


def pct(xs, q):
    return xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]


def attn_bound_us(m):
    """max(bytes / HBM peak, flops / bf16 MFMA peak) of one attention launch."""
    return max(m["attn_bytes"] / (HBM_PEAK_GBS * 1e3), m["attn_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e6))


def workload_entry(m):
    """One workload of the per-workload object: round time, rows/s, the
    attention launch against its HBM roofline and its max(bytes/BW,
    flops/peak) bound, and the attention + merge pair."""
    a_gbs = m["attn_bytes"] / (m["attn_us"] * 1e-6) / 1e9
    pair_bytes = m["attn_bytes"] + m["merge_bytes"]
    bound = attn_bound_us(m)
    return {
        "rows": m["R"], "streams": m["S"], "sum_keys": m["sum_keys"],
        "rows_per_s": m["R"] / (m["ms_step"] * 1e-3), "round_ms": m["ms_step"],
        "eager_round_ms_median": m["round_ms"][len(m["round_ms"]) // 2],
        "attn_us": m["attn_us"], "attn_gbs": a_gbs, "attn_frac_hbm": a_gbs / HBM_PEAK_GBS,
        "attn_flops": m["attn_flops"], "attn_bound_us": bound, "attn_frac_of_bound": bound / m["attn_us"],
        "attn_merge_us": m["pair_us"],
        "attn_merge_frac_hbm": pair_bytes / (m["pair_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "attn_graph_us": m["attn_graph_us"],
        "attn_graph_frac_hbm": (None if m["attn_graph_us"] is None
                                else m["attn_bytes"] / (m["attn_graph_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch

    import attention_stream_verify_amd as asv
    import workloads

    asv.lib()  # fails loudly when libasv.so is missing
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    m = measure_round(torch, asv, workloads, dev, args.config, args.steps, args.warmup,
                      block=args.block, with_qk=args.with_qk, eager=args.eager, seed=args.seed)
    rnd, rb, R, S = m["rnd"], m["rb"], m["R"], m["S"]
    attn_bytes, attn_flops, merge_bytes = m["attn_bytes"], m["attn_flops"], m["merge_bytes"]
    attn_avg_ms, pair_avg_ms = m["attn_us"] * 1e-3, m["pair_us"] * 1e-3
    achieved = attn_bytes / (attn_avg_ms * 1e-3) / 1e9
    qkv, gq, gk = m["qkv"]
    round_ms = m["round_ms"]

    # draft-id gather over the round's picks, queued behind an attention
    # launch like the qk leg below, so the events time the kernels
    rb.draft()
    rb.attn(0, rnd.attn[0][0])
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    for _ in range(16):
        rb.draft()
    d1.record()
    torch.cuda.synchronize()
    draft_us = d0.elapsed_time(d1) * 1e3 / 16

    markov = None if args.no_markov else markov_leg(torch, asv, dev, rnd.seed)

    # The qk stage alone: its launches are queued behind an attention launch
    # (which runs far longer than the host needs to enqueue them), so the GPU
    # runs them back to back and the events time the kernels, not the
    # Python calls. One launch per attention layer, three passes.
    qk_us = []
    for _ in range(3):
        rb.attn(0, rnd.attn[0][0])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(rnd.n_attn):
            rb.qk(i, qkv, gq, gk, workloads.ROPE_THETA, workloads.NORM_EPS)
        b.record()
        torch.cuda.synchronize()
        qk_us.append(a.elapsed_time(b) * 1e3 / rnd.n_attn)
    qk_avg = sorted(qk_us)[1]

    # host table build, timed on its own (pure host code, no HIP calls)
    from attention_stream_verify_amd import _lib
    build_us = _lib.time_table_build(rnd.streams, [layer[2] for layer in rnd.conv],
                                     [layer[1] for layer in rnd.attn],
                                     [layer[2] for layer in rnd.attn], full=args.block)

    line = {
        "metric": ("verify rows/sec per shared round (conv+qk+attn+argmax); attn HBM GB/s vs peak"
                   if args.with_qk else
                   "verify rows/sec per shared round (conv+attn+argmax); attn HBM GB/s vs peak"),
        "value": R / (m["ms_step"] * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[args.config] + (", block (non-causal) attention"
                                                        if args.block else "")
                        + (", qk stage before every attention layer" if args.with_qk else ""),
            "streams": S,
            "rows": R,
            "sum_keys": m["sum_keys"],
            "conv_layers": rnd.n_conv,
            "attn_layers": rnd.n_attn,
            "vocab": int(rnd.logits.shape[1]),
            "seed": rnd.seed,
        },
        "roofline": {
            "kernel": "attn_split (asv_shared_attn)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None if args.block else profiled_traffic(args.config),
            "bytes_per_launch": attn_bytes,
            "flops_per_launch": attn_flops,
            "mfma_frac": attn_flops / (attn_avg_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "avg_launch_us": attn_avg_ms * 1e3,
            # the same launches replayed from a captured graph (no host latency)
            "graph_avg_launch_us": m["attn_graph_us"],
        },
        "launch": "eager" if args.eager else "hip graph of one round",
        "eager_ms_per_step": m["eager_ms_step"],
        "round_ms": {"median": round_ms[len(round_ms) // 2], "p10": pct(round_ms, 0.1),
                     "p90": pct(round_ms, 0.9)},
        "attn_merge": {
            "bytes_per_layer": attn_bytes + merge_bytes,
            "avg_pair_us": pair_avg_ms * 1e3,
            "achieved_gbs": (attn_bytes + merge_bytes) / (pair_avg_ms * 1e-3) / 1e9,
            "frac": (attn_bytes + merge_bytes) / (pair_avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        },
        "mfma_busy": None if args.block else profiled_mfma(args.config),
        "table_build_host_us": build_us,
        "draft_ids_us": draft_us,
        "markov": markov,
        "qk": {"avg_launch_us": qk_avg, "bytes_per_launch": R * (2 * 3072 + 2 * 2048 + 2 * 512 + 2 * 512) + 2 * 128,
               "achieved_gbs": (R * (2 * 3072 + 2 * 2048 + 2 * 512 + 2 * 512) + 2 * 128) / (qk_avg * 1e-6) / 1e9,
               "in_round": bool(args.with_qk)},
        "workloads": None,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(rnd, R, full=args.block)
        line["cpu_baseline"]["gpu_over_cpu"] = line["value"] / line["cpu_baseline"]["value"]

    # every workload, measured in this run the same way (the default
    # workload's own numbers are reused for its entry)
    if not args.no_workloads:
        entries = {}
        del rnd, rb
        m_self = workload_entry(m)
        m_self.update({"mfma_busy": line["mfma_busy"], "traffic_bytes": line["roofline"]["traffic"]})
        del m
        for c in range(5):
            if c == args.config and not args.block and not args.with_qk:
                entries[WORKLOAD_KEYS[c]] = m_self
                continue
            mc = measure_round(torch, asv, workloads, dev, c, args.workload_steps, args.warmup,
                               block=args.block, with_qk=args.with_qk, eager=args.eager)
            e = workload_entry(mc)
            e["mfma_busy"] = None if args.block else profiled_mfma(c)
            e["traffic_bytes"] = None if (args.block or args.with_qk) else profiled_traffic(c)
            entries[WORKLOAD_KEYS[c]] = e
            del mc
            torch.cuda.empty_cache()
        line["workloads"] = entries
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
