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
* split plan: the splits depend only on the stream's own rows and keys (so
  a shared round gives the same bits as each stream alone): with
  wt = min(w_s, 16), the cap C_s = 768 (wt <= 2), 1024 (wt <= 4),
  2560 (wt <= 8), 7168 (otherwise), and 5120 for a stream of more than 16
  rows (a prompt chunk), the keys are cut into
  n_s = ceil(K_s / C_s) consecutive splits, each starting at a multiple of
  32 keys, the last one ending at K_s:
  - equal splits (wt <= 8, or n_s = 1): size S_s = ceil(K_s / n_s) rounded
    up to a multiple of 32 (so S_s <= C_s and ceil(K_s / S_s) = n_s);
  - otherwise two sizes: the first b_s = ceil(n_s / 2) splits of A_s keys,
    A_s = ceil(5 K_s / (5 b_s + 4 (n_s - b_s))) rounded up to 32, and the
    rest of B_s = ceil((K_s - b_s A_s) / (n_s - b_s)) keys rounded up to 32
    (about 4/5 of A_s; falling back to equal splits if that left a split
    empty, which no admitted key count does);
* partial records: stream s owns records [poff_s, poff_s + nsplit_s*w_s*32),
  poff being the exclusive prefix sum of nsplit_s*w_s*32; the record of
  (row r, q head h, split t) is poff_s + (t*w_s + pos_r)*32 + h;
* work items: a stream of one tile has an item for every kv head and split
  that holds a key the tile's last row can see; a longer stream (a prompt
  chunk) is cut into groups of up to 4 consecutive tiles (the last group
  shorter), each group an item for every kv head and split that holds a key
  the last row of its last tile can see. An item is (first tile, kv head,
  split, tiles in it).

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
GROUP_TILES = 4
N_Q_HEADS = 32
N_KV_HEADS = 8
KEY_BLOCK = 32
MAX_ROWS = 2048
MAX_KEYS = 131072


def split_cap(rows):
    """Largest split C_s for a stream of ``rows`` window rows."""
    if int(rows) > TILE_ROWS:
        return 5120
    wt = min(int(rows), TILE_ROWS)
    if wt <= 2:
        return 768
    if wt <= 4:
        return 1024
    if wt <= 8:
        return 2560
    return 7168


def _up32(x):
    return -(-int(x) // 32) * 32


def split_plan(rows, keys):
    """(A, B, b, n): n splits, the first b of A keys and the rest of B keys
    (equal splits: A = B and b = n)."""
    K = int(keys)
    n = -(-K // split_cap(rows))
    equal = _up32(-(-K // n))
    if min(int(rows), TILE_ROWS) <= 8 or n == 1:
        return equal, equal, n, n
    b = -(-n // 2)
    A = _up32(-(-5 * K // (5 * b + 4 * (n - b))))
    rest = K - b * A
    B = _up32(-(-rest // (n - b))) if rest > 0 else 0
    if rest <= 0 or b * A + (n - b - 1) * B >= K:
        return equal, equal, n, n
    return A, B, b, n


def split_bounds(rows, keys):
    """Start key of every split, then K_s: split t covers [bounds[t], bounds[t+1])."""
    A, B, b, n = split_plan(rows, keys)
    starts = [t * A for t in range(b)] + [b * A + t * B for t in range(n - b)]
    return np.array(starts + [int(keys)], dtype=np.int64)


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
    split: np.ndarray           # A_s (S_s for equal splits)
    nsplit: np.ndarray          # n_s
    split_tail: np.ndarray      # B_s
    nbig: np.ndarray            # b_s
    bounds: list                # per stream: split starts, then K_s
    poff: np.ndarray            # S (int64)
    partial_count: int
    work: np.ndarray            # [n_work, 4]: first tile, kv head, split, tiles
    n_rows: int = field(default=0)

    def record(self, r, h, t):
        s = int(self.row_stream[r])
        return int(self.poff[s]) + (t * int(self.rows[s]) + int(self.row_pos[r])) * N_Q_HEADS + h

    def splits_before(self, s, n):
        """Splits of stream s that start below key n (hold a key of [0, n))."""
        return int(np.count_nonzero(self.bounds[s][:-1] < int(n)))

    def row_nsplit(self, r):
        """Splits holding at least one key row r sees."""
        return self.splits_before(int(self.row_stream[r]), self.row_nkeys[r])

    def split_range(self, s, t):
        """Keys [lo, hi) of split t of stream s."""
        return int(self.bounds[s][t]), int(self.bounds[s][t + 1])


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

    plans = [split_plan(rows[s], keys[s]) for s in range(S)]
    split = np.array([p[0] for p in plans], dtype=np.int64)
    split_tail = np.array([p[1] for p in plans], dtype=np.int64)
    nbig = np.array([p[2] for p in plans], dtype=np.int64)
    nsplit = np.array([p[3] for p in plans], dtype=np.int64)
    bounds = [split_bounds(rows[s], keys[s]) for s in range(S)]
    poff = np.zeros(S, dtype=np.int64)
    acc = 0
    for s in range(S):
        poff[s] = acc
        acc += int(nsplit[s] * rows[s] * N_Q_HEADS)
    partial_count = acc

    work = []
    for s in range(S):
        mine = [ti for ti in range(len(tiles)) if tiles[ti][0] == s]
        groups = [mine] if len(mine) == 1 else \
            [mine[i:i + GROUP_TILES] for i in range(0, len(mine), GROUP_TILES)]
        for grp in groups:
            _s, _r0, n, p0 = tiles[grp[-1]]
            n_last = keys[s] if full else keys[s] - rows[s] + p0 + n
            for t in range(int(np.count_nonzero(bounds[s][:-1] < n_last))):
                for g in range(N_KV_HEADS):
                    work.append((grp[0], g, t, len(grp)))
    work = np.array(work, dtype=np.int64).reshape(-1, 4)

    return Table(rows=rows, keys=keys, caps=caps, seg_off=seg_off, row_stream=row_stream,
                 row_pos=row_pos, row_nkeys=row_nkeys, tiles=tiles, split=split,
                 nsplit=nsplit, split_tail=split_tail, nbig=nbig, bounds=bounds, poff=poff,
                 partial_count=partial_count, work=work, n_rows=R)
