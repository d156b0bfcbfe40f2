"""Seeded synthetic inputs for the shared-round verify step.

This module draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the oracle-side tests and the GPU path take their
inputs from here.

The pages' workloads are served prompts on a real checkpoint (absent here);
these seeded shapes stand in for them. Five workloads are defined, sized as
the pages' served rounds (16-stream decode rounds, draft windows up to 16
rows, contexts up to 131,072 keys, a 2,048-row scratch):

0. tiny: 4 streams, windows {1,2,3,4}, keys {16,64,128,256}; 1 conv + 1 attn
   layer; logits with planted ties and one NaN row.
1. decode: 16 streams x 1 row, keys uniform in 512..4096; 30 conv + 10 attn
   layers; 1% tie positions per logit row.
2. verify: 16 streams x 8 rows, keys log-uniform in 2048..32768; one +Inf
   row and one NaN row.
3. long: 4 streams x 16 rows, keys {65536, 98304, 130816, 131072}.
4. scratch: 48 streams with windows uniform in 1..16 and lognormal keys
   (median 8192, sigma 1, clipped to [rows, 131072]), plus prompt chunks of
   512 rows (the last one shorter) up to 2,048 rows; 1% tie positions in every
   16th logit row and 8 nonfinite rows.

Value distributions: Q, K, V, X and conv states ~ N(0, 1); conv weights
~ N(0, 1)/sqrt(3); logits ~ N(0, sigma=3). Draws are float32 rounded to bf16
(round to nearest even) and kept as uint16 bit patterns (torch.int16 views on
the device). Cache slots past a stream's key count hold NaN, so a read past
the count shows up.

Cache layouts (the library's device layout):
* K: [8 kv heads][capacity][64] bf16, key-major;
* V: [8 kv heads][capacity/32][64][32] bf16: blocks of 32 keys, each block
  stored d-major (64 rows of 32 consecutive keys).
``v_logical`` / ``v_blocked`` convert between V's logical [8][keys][64] and
that layout (a pure index permutation).
"""

import math

import numpy as np
import torch

HIDDEN = 2048
CONV_IN = 6144
N_Q = 32
N_KV = 8
D = 64
VOCAB = 128000
KEY_BLOCK = 32
MAX_KEYS = 131072

NAMES = ["tiny", "decode", "verify", "long", "scratch"]
LAYERS = {0: (1, 1), 1: (30, 10), 2: (30, 10), 3: (30, 10), 4: (30, 10)}


def round_up(x, m):
    return ((x + m - 1) // m) * m


def capacity(keys):
    """Cache capacity of a stream: its key count rounded up to 256 slots."""
    return min(round_up(keys, 256), MAX_KEYS)


# ----------------------------------------------------------------- streams

def streams_for(config, seed=None):
    """Stream descriptors [(rows, keys, capacity)] of a workload."""
    seed = config if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    if config == 0:
        rk = [(1, 16), (2, 64), (3, 128), (4, 256)]
    elif config == 1:
        rk = [(1, int(k)) for k in rng.integers(512, 4097, size=16)]
    elif config == 2:
        ks = np.exp(rng.uniform(math.log(2048), math.log(32768), size=16))
        rk = [(8, int(round(k))) for k in ks]
    elif config == 3:
        rk = [(16, 65536), (16, 98304), (16, 130816), (16, 131072)]
    elif config == 4:
        ws = rng.integers(1, 17, size=48)
        rk = []
        for w in ws:
            k = int(round(8192.0 * math.exp(rng.standard_normal())))
            rk.append((int(w), int(min(max(k, w), MAX_KEYS))))
        left = 2048 - sum(w for w, _ in rk)
        while left > 0:
            c = min(512, left)
            k = int(round(8192.0 * math.exp(rng.standard_normal())))
            rk.append((c, int(min(max(k, c), MAX_KEYS))))
            left -= c
    else:
        raise ValueError(f"unknown workload {config}")
    return [(w, k, capacity(k)) for (w, k) in rk]


# ------------------------------------------------------------ tensor draws

def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _bf16_normal(shape, g, device, std=1.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(torch.bfloat16).view(torch.int16)


_NAN_BF16 = 0x7FC0


def kv_cache(keys, cap, g, device):
    """One stream's K and V (device layout) with NaN past the key count."""
    k = _bf16_normal((N_KV, cap, D), g, device)
    v = _bf16_normal((N_KV, cap, D), g, device)
    if cap > keys:
        k[:, keys:, :] = _NAN_BF16
        v[:, keys:, :] = _NAN_BF16
    return k.contiguous(), v_blocked(v)


def v_blocked(v_logical_t):
    """[8][cap][64] -> [8][cap/32][64][32] (d-major inside 32-key blocks)."""
    h, cap, d = v_logical_t.shape
    assert cap % KEY_BLOCK == 0
    return v_logical_t.reshape(h, cap // KEY_BLOCK, KEY_BLOCK, d).transpose(2, 3).contiguous()


def v_logical(v_blk):
    """[8][cap/32][64][32] -> [8][cap][64]."""
    h, nb, d, kb = v_blk.shape
    return v_blk.transpose(2, 3).reshape(h, nb * kb, d).contiguous()


def conv_layer(R, S, g, device):
    X = _bf16_normal((R, CONV_IN), g, device)
    W = _bf16_normal((HIDDEN, 3), g, device, std=1.0 / math.sqrt(3.0))
    states = [_bf16_normal((2, HIDDEN), g, device) for _ in range(S)]
    return X, W, states


def attn_layer(streams, g, device):
    R = sum(w for w, _, _ in streams)
    Q = _bf16_normal((R, N_Q, D), g, device)
    ks, vs = [], []
    for (_, k, cap) in streams:
        kk, vv = kv_cache(k, cap, g, device)
        ks.append(kk)
        vs.append(vv)
    return Q, ks, vs


# qk stage constants: the pages give neither; these are stand-ins of the
# usual size for this model family.
ROPE_THETA = 1.0e6
NORM_EPS = 1.0e-5


def qk_inputs(R, seed, device):
    """One attention layer's qk-stage inputs: the rows' qkv projections
    ~ N(0, 1) and the q and k norm gains ~ 1 + N(0, 0.1^2), as bf16 bits."""
    g = _gen(device, seed)
    qkv = _bf16_normal((R, (N_Q + 2 * N_KV) * D), g, device)
    gains = []
    for _ in range(2):
        x = 1.0 + 0.1 * torch.randn((D,), generator=g, device=device, dtype=torch.float32)
        gains.append(x.to(torch.bfloat16).view(torch.int16))
    return qkv, gains[0], gains[1]


def logits_for(config, R, g, device, vocab=VOCAB):
    """bf16 logits ~ N(0, 3) with the workload's planted ties and nonfinite rows.

    Returns (logits int16 [R][vocab], notes) where notes lists what was planted.
    Planting uses a host NumPy generator seeded from the torch draw so that the
    positions do not depend on the device.
    """
    L = _bf16_normal((R, vocab), g, device, std=3.0)
    seed = int(torch.randint(0, 2**31 - 1, (1,), generator=g, device=device).item())
    rng = np.random.Generator(np.random.PCG64(seed))
    notes = []
    NAN, PINF, NINF = _NAN_BF16, 0x7F80, -128  # 0xFF80 as int16

    def row_max_pos(r):
        v = L[r].view(torch.bfloat16).float()
        return int(torch.argmax(v).item())

    if config == 0:
        higher_row = int(rng.integers(0, R))
        nan_row = int(rng.integers(0, R))
        for r in range(R):
            a = row_max_pos(r)
            if r == higher_row and a + 1 < vocab:
                b = int(rng.integers(a + 1, vocab))
            elif a > 0:
                b = int(rng.integers(0, a))
            else:
                continue
            L[r, b] = L[r, a].clone()
            notes.append(("tie", r, a, b))
        pos = int(rng.integers(0, vocab))
        L[nan_row, pos] = NAN
        notes.append(("nan", nan_row, pos))
    elif config in (1, 4):
        rows = range(R) if config == 1 else range(0, R, 16)
        nt = vocab // 100
        for r in rows:
            a = row_max_pos(r)
            pos = torch.from_numpy(rng.choice(vocab, size=nt, replace=False)).to(device)
            L[r, pos] = L[r, a].clone()
            notes.append(("ties", r, nt))
        if config == 4:
            bad = rng.choice(R, size=8, replace=False)
            kinds = ["nan", "pinf", "ninf", "mixed", "nan", "pinf", "ninf", "mixed"]
            for r, kind in zip(bad.tolist(), kinds):
                p = int(rng.integers(0, vocab))
                if kind == "nan":
                    L[r, p] = NAN
                elif kind == "pinf":
                    L[r, p] = PINF
                elif kind == "ninf":
                    L[r, p] = NINF
                else:
                    L[r, p] = NAN
                    L[r, (p + 7) % vocab] = PINF
                    L[r, (p + 13) % vocab] = NINF
                notes.append((kind, r, p))
    elif config == 2:
        r_inf, r_nan = rng.choice(R, size=2, replace=False).tolist()
        L[r_inf, int(rng.integers(0, vocab))] = PINF
        L[r_nan, int(rng.integers(0, vocab))] = NAN
        notes += [("pinf", r_inf), ("nan", r_nan)]
    return L, notes


class Round:
    """All inputs of one shared round of a workload, on one device."""

    def __init__(self, config, device="cpu", seed=None, n_conv=None, n_attn=None,
                 streams=None, vocab=VOCAB, with_logits=True):
        self.config = config
        self.seed = config if seed is None else seed
        self.streams = streams if streams is not None else streams_for(config, self.seed)
        dc, da = LAYERS.get(config, (1, 1))
        self.n_conv = dc if n_conv is None else n_conv
        self.n_attn = da if n_attn is None else n_attn
        self.R = sum(w for w, _, _ in self.streams)
        self.S = len(self.streams)
        g = _gen(device, self.seed)
        self.conv = [conv_layer(self.R, self.S, g, device) for _ in range(self.n_conv)]
        self.attn = [attn_layer(self.streams, g, device) for _ in range(self.n_attn)]
        if with_logits:
            self.logits, self.notes = logits_for(config, self.R, g, device, vocab)
        else:
            self.logits, self.notes = None, []
