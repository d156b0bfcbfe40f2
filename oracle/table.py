"""Segment table of a shared round (oracle; test infrastructure only).

PR #1377 "LFM2: shared-round decode", the shared-round commit of the commit
log and the "What this changes" list: a shared round runs each layer once
over every row of every stream, through a table of the streams' cache
addresses, row offsets and key counts; the table also gives a row map and
tiles; the scratch keeps each stream's attention partials apart. The pages
print no layout for any of it, so the arrays below are this oracle's own
definitions (the readings are listed in the design notes):

* streams are taken in caller order; stream s has w_s rows, K_s keys in its
  cache (K_s counts the window's own keys) and a cache capacity cap_s;
* row offsets: off_0 = 0, off_{s+1} = off_s + w_s;
* row map: row r in [off_s, off_s + w_s) has stream s and position
  pos = r - off_s, and sees n_r = K_s - w_s + pos + 1 keys (causal inside the
  window);
* tiles: runs of at most 16 consecutive rows, never across streams;
* split plan: the split size depends only on the stream's own rows and
  keys (so a shared round gives the same bits as each stream alone): with
  wt = min(w_s, 16), the cap C_s = 512 (wt <= 2), 1024 (wt <= 4),
  2048 (wt <= 8), 7168 (otherwise); the keys are cut into
  n_s = ceil(K_s / C_s) equal splits, S_s = ceil(K_s / n_s) rounded up to a
  multiple of 32 (so S_s <= C_s and nsplit_s = ceil(K_s / S_s) = n_s);
* partial records: stream s owns records [poff_s, poff_s + nsplit_s*w_s*32),
  poff being the exclusive prefix sum of nsplit_s*w_s*32; the record of
  (row r, q head h, split t) is poff_s + (t*w_s + pos_r)*32 + h;
* work items: for every tile, kv head and split that holds a key the tile's
  last row can see.

Block mode (PR #1391 "lfm2: draft with LiquidAI's DSpark drafter
(--drafter)", its list of new kernels: the target's attention and merge with
a FULL flag, every block row seeing the keys [0, len + 1)): read as every row
of a stream seeing all of its K_s keys, n_r = K_s, so the window's rows
attend to each other both ways; the work items then cover every split of
the stream for every tile. Everything else is as above.
"""

from dataclasses import dataclass, field

import numpy as np

TILE_ROWS = 16
N_Q_HEADS = 32
N_KV_HEADS = 8
KEY_BLOCK = 32
MAX_ROWS = 2048
MAX_KEYS = 131072


def split_cap(rows):
    """Largest split C_s for a stream of ``rows`` window rows."""
    wt = min(int(rows), TILE_ROWS)
    if wt <= 2:
        return 512
    if wt <= 4:
        return 1024
    if wt <= 8:
        return 2048
    return 7168


def split_keys(rows, keys):
    """Split size S_s: K_s keys cut into ceil(K_s / C_s) equal splits, each
    rounded up to a multiple of 32 keys."""
    cap = split_cap(rows)
    n = -(-int(keys) // cap)
    s = -(-int(keys) // n)
    return -(-s // 32) * 32


@dataclass
class Table:
    rows: np.ndarray            # w_s
    keys: np.ndarray            # K_s
    caps: np.ndarray            # cap_s
    seg_off: np.ndarray         # S+1
    row_stream: np.ndarray      # R
    row_pos: np.ndarray         # R
    row_nkeys: np.ndarray       # R
    tiles: np.ndarray           # [n_tiles, 4]: stream, first row, row count, first pos
    split: np.ndarray           # S_s
    nsplit: np.ndarray          # nsplit_s
    poff: np.ndarray            # S (int64)
    partial_count: int
    work: np.ndarray            # [n_work, 3]: tile, kv head, split
    n_rows: int = field(default=0)

    def record(self, r, h, t):
        s = int(self.row_stream[r])
        return int(self.poff[s]) + (t * int(self.rows[s]) + int(self.row_pos[r])) * N_Q_HEADS + h

    def row_nsplit(self, r):
        """Splits holding at least one key row r sees."""
        s = int(self.row_stream[r])
        return -(-int(self.row_nkeys[r]) // int(self.split[s]))


def validate(streams):
    """Raise ValueError unless the stream descriptors form a valid round."""
    if len(streams) < 1:
        raise ValueError("no streams")
    total = 0
    for (w, k, cap) in streams:
        if w < 1:
            raise ValueError("a stream needs at least one row")
        if k < w:
            raise ValueError("key count below the window's rows")
        if k > MAX_KEYS:
            raise ValueError("key count above 131072")
        if cap < k or cap % KEY_BLOCK != 0 or cap > MAX_KEYS:
            raise ValueError("capacity must hold the keys, be a multiple of 32 and at most 131072")
        total += w
    if total > MAX_ROWS:
        raise ValueError("more than 2048 rows")


def build(streams, full=False):
    """streams: sequence of (rows, key_count, kv_capacity) in caller order;
    full: block mode (every row sees all of its stream's keys)."""
    validate(streams)
    S = len(streams)
    rows = np.array([s[0] for s in streams], dtype=np.int64)
    keys = np.array([s[1] for s in streams], dtype=np.int64)
    caps = np.array([s[2] for s in streams], dtype=np.int64)

    seg_off = np.zeros(S + 1, dtype=np.int64)
    for s in range(S):
        seg_off[s + 1] = seg_off[s] + rows[s]
    R = int(seg_off[S])

    row_stream = np.zeros(R, dtype=np.int64)
    row_pos = np.zeros(R, dtype=np.int64)
    row_nkeys = np.zeros(R, dtype=np.int64)
    for s in range(S):
        for i in range(rows[s]):
            r = seg_off[s] + i
            row_stream[r] = s
            row_pos[r] = i
            row_nkeys[r] = keys[s] if full else keys[s] - rows[s] + i + 1

    tiles = []
    for s in range(S):
        p = 0
        while p < rows[s]:
            n = min(TILE_ROWS, rows[s] - p)
            tiles.append((s, seg_off[s] + p, n, p))
            p += n
    tiles = np.array(tiles, dtype=np.int64).reshape(-1, 4)

    split = np.array([split_keys(rows[s], keys[s]) for s in range(S)], dtype=np.int64)
    nsplit = np.array([-(-keys[s] // split[s]) for s in range(S)], dtype=np.int64)
    poff = np.zeros(S, dtype=np.int64)
    acc = 0
    for s in range(S):
        poff[s] = acc
        acc += int(nsplit[s] * rows[s] * N_Q_HEADS)
    partial_count = acc

    work = []
    for ti, (s, _r0, n, p0) in enumerate(tiles):
        n_last = keys[s] if full else keys[s] - rows[s] + p0 + n
        for t in range(-(-int(n_last) // int(split[s]))):
            for g in range(N_KV_HEADS):
                work.append((ti, g, t))
    work = np.array(work, dtype=np.int64).reshape(-1, 3)

    return Table(rows=rows, keys=keys, caps=caps, seg_off=seg_off, row_stream=row_stream,
                 row_pos=row_pos, row_nkeys=row_nkeys, tiles=tiles, split=split,
                 nsplit=nsplit, poff=poff, partial_count=partial_count, work=work, n_rows=R)
