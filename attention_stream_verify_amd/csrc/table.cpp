// Segment table of a shared round: host code, no HIP calls.
//
// PR #1377 "LFM2: shared-round decode", shared-round commit: each layer runs
// once over every row of every live stream, driven by one per-stream table
// (where each stream's caches live, where its rows start, how many keys it
// holds); the table carries a row map and tiles, and each stream's attention
// partials get a range of their own.
// The layout of every array is given in include/asv.h.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <utility>
#include <vector>

#include "asv.h"

namespace {

// Split plan of one stream, from its own rows and keys only (so a shared
// round gives the same bits as each stream alone): n = ceil(keys / cap)
// consecutive splits, each starting at a multiple of 32 keys. Few short
// windows make many small splits (one- and two-row windows: at most 768
// keys, which puts a 16-stream decode round with 512-4,096 keys in one
// round of the device's 512 resident blocks; windows of 5 to 8 rows: at most 2,560
// keys, which puts the 16 x 8-row verify round's 472 items in one round too,
// where 1,024-2,304 and 3,072 were slower); 16-row tiles take splits of about 7,168
// keys, which at 131,072-key contexts puts one tile's 8 heads x 19 splits,
// and four such streams' 496 work items, on the 512 blocks the device holds
// at once. Prompt chunks (streams of more than one tile) take at most 5,120
// keys a split: their group items are arithmetic-bound, and shorter ones
// end closer together.
//
// Windows of up to 8 rows cut their keys into n equal splits. 16-row tiles
// take two sizes, the first ceil(n / 2) splits 5/4 the size of the rest:
// the work list runs the larger items first, so on a device holding two
// blocks a CU each CU pairs a larger item with a smaller one, and the block
// dispatched first, which streams faster (its waves win issue), has the
// larger share; the two then finish together instead of the second block
// running alone at the end.
int32_t split_cap(int32_t rows) {
  if (rows > ASV_TILE_ROWS) return 5120;  // prompt chunks
  const int32_t wt = rows < ASV_TILE_ROWS ? rows : ASV_TILE_ROWS;
  if (wt <= 2) return 768;
  if (wt <= 4) return 1024;
  if (wt <= 8) return 2560;
  return 7168;
}

int32_t up32(int64_t x) { return int32_t((x + 31) / 32 * 32); }

struct Plan {
  int32_t a, b, nbig, n;  // n splits: nbig of a keys, then b keys
};

Plan split_plan(int32_t rows, int32_t keys) {
  const int32_t n = (keys + split_cap(rows) - 1) / split_cap(rows);
  const int32_t eq = up32((int64_t(keys) + n - 1) / n);
  const Plan equal{eq, eq, n, n};
  if ((rows < ASV_TILE_ROWS ? rows : ASV_TILE_ROWS) <= 8 || n == 1) return equal;
  const int32_t nb = (n + 1) / 2;
  const int64_t den = 5 * int64_t(nb) + 4 * int64_t(n - nb);
  const int32_t a = up32((5 * int64_t(keys) + den - 1) / den);
  const int64_t rest = int64_t(keys) - int64_t(nb) * a;
  if (rest <= 0) return equal;
  const int32_t b = up32((rest + (n - nb) - 1) / (n - nb));
  if (int64_t(nb) * a + int64_t(n - nb - 1) * b >= keys) return equal;  // an empty split
  return Plan{a, b, nb, n};
}

int32_t split_start(const Plan& p, int32_t t) {
  return t < p.nbig ? t * p.a : p.nbig * p.a + (t - p.nbig) * p.b;
}

static_assert(sizeof(asv_seg) == 48, "asv_seg layout");
static_assert(sizeof(asv_work) == 16, "asv_work layout");
// every stream holds a row, so a stream index fits asv_work's int16 field
static_assert(ASV_MAX_ROWS <= 32767, "asv_work stream field");

// Tiles of one group item (one a wave of the attention block).
constexpr int32_t kGroupTiles = 4;
// Work-list runs: 256 blocks, one a CU of the device, dispatched first.
constexpr size_t kRun = 256;

int64_t align16(int64_t x) { return (x + 15) & ~int64_t(15); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// True when the byte ranges [p, p + n) overlap pairwise for no two entries.
bool disjoint(std::vector<std::pair<uintptr_t, uintptr_t>>& spans) {
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second) return false;
  return true;
}

}  // namespace

extern "C" int asv_abi_version(void) { return ASV_ABI_VERSION; }

extern "C" const char* asv_strerror(int code) {
  switch (code) {
    case ASV_OK: return "ok";
    case ASV_E_ARG: return "null, misaligned or aliasing pointer";
    case ASV_E_SHAPE: return "rows, keys, capacity or layer out of range";
    case ASV_E_UNSUPPORTED: return "dimension other than the compiled one";
    case ASV_E_CAPACITY: return "caller buffer too small";
    case ASV_E_HIP: return "HIP runtime refused a copy or launch";
    default: return "unknown error code";
  }
}

namespace {

// full: block mode, every row seeing all of its stream's keys.
int build_table(const asv_stream_desc* streams, int32_t n_streams, const void* const* conv_state,
                int32_t n_conv_layers, const void* const* k_cache, const void* const* v_cache,
                int32_t n_attn_layers, void* blob, size_t blob_bytes, asv_table_info* info,
                bool full) {
  if (streams == nullptr || info == nullptr) return ASV_E_ARG;
  if (n_streams < 1 || n_conv_layers < 0 || n_attn_layers < 0) return ASV_E_SHAPE;

  // ---- descriptors
  int64_t total_rows = 0;
  for (int32_t s = 0; s < n_streams; ++s) {
    const asv_stream_desc& d = streams[s];
    if (d.rows < 1 || d.key_count < d.rows || d.key_count > ASV_MAX_KEYS) return ASV_E_SHAPE;
    if (d.kv_capacity < d.key_count || d.kv_capacity > ASV_MAX_KEYS ||
        d.kv_capacity % ASV_KEY_BLOCK != 0)
      return ASV_E_SHAPE;
    total_rows += d.rows;
    if (total_rows > ASV_MAX_ROWS) return ASV_E_SHAPE;
  }
  const int32_t S = n_streams;
  const int32_t R = static_cast<int32_t>(total_rows);

  // ---- addresses: present, aligned, and no two streams sharing bytes
  if (n_conv_layers > 0 && conv_state == nullptr) return ASV_E_ARG;
  if (n_attn_layers > 0 && (k_cache == nullptr || v_cache == nullptr)) return ASV_E_ARG;
  const uintptr_t state_bytes = 2u * ASV_HIDDEN * sizeof(uint16_t);
  std::vector<std::pair<uintptr_t, uintptr_t>> spans;
  for (int32_t l = 0; l < n_conv_layers; ++l) {
    spans.clear();
    for (int32_t s = 0; s < S; ++s) {
      const void* p = conv_state[int64_t(l) * S + s];
      if (p == nullptr || !aligned16(p)) return ASV_E_ARG;
      const uintptr_t a = reinterpret_cast<uintptr_t>(p);
      spans.emplace_back(a, a + state_bytes);
    }
    if (!disjoint(spans)) return ASV_E_ARG;
  }
  for (int32_t l = 0; l < n_attn_layers; ++l) {
    spans.clear();
    for (int32_t s = 0; s < S; ++s) {
      const uintptr_t bytes =
          uintptr_t(ASV_KV_HEADS) * uintptr_t(streams[s].kv_capacity) * ASV_HEAD_DIM * sizeof(uint16_t);
      for (const void* const* arr : {k_cache, v_cache}) {
        const void* p = arr[int64_t(l) * S + s];
        if (p == nullptr || !aligned16(p)) return ASV_E_ARG;
        const uintptr_t a = reinterpret_cast<uintptr_t>(p);
        spans.emplace_back(a, a + bytes);
      }
    }
    if (!disjoint(spans)) return ASV_E_ARG;
  }

  // ---- segments, rows, tiles, split plan, partial ranges
  std::vector<asv_seg> segs(S);
  std::vector<asv_row> rows(R);
  std::vector<asv_tile> tiles;
  int64_t poff = 0;
  int32_t row0 = 0;
  int32_t max_tile_rows = 0;
  for (int32_t s = 0; s < S; ++s) {
    const asv_stream_desc& d = streams[s];
    asv_seg& g = segs[s];
    g.row0 = row0;
    g.rows = d.rows;
    g.keys = d.key_count;
    g.cap = d.kv_capacity;
    const Plan pl = split_plan(d.rows, d.key_count);
    g.split_keys = pl.a;
    g.nsplit = pl.n;
    g.split_tail = pl.b;
    g.nbig = pl.nbig;
    g.poff = poff;
    poff += int64_t(g.nsplit) * d.rows * ASV_Q_HEADS;
    for (int32_t p = 0; p < d.rows; p += ASV_TILE_ROWS) {
      asv_tile t;
      t.stream = s;
      t.row0 = row0 + p;
      t.nrows = std::min(ASV_TILE_ROWS, d.rows - p);
      t.pos0 = p;
      max_tile_rows = std::max(max_tile_rows, t.nrows);
      for (int32_t i = 0; i < t.nrows; ++i) {
        asv_row& r = rows[t.row0 + i];
        r.stream = s;
        r.pos = p + i;
        r.nkeys = full ? d.key_count : d.key_count - d.rows + p + i + 1;
        r.tile = static_cast<int32_t>(tiles.size());
      }
      tiles.push_back(t);
    }
    row0 += d.rows;
  }

  // ---- attention work: (tiles, kv head, split) for every split holding a
  // key the last row of the item's last tile sees. A stream of one tile is
  // one item a split and head; a longer stream (a prompt chunk) is cut into
  // groups of up to kGroupTiles consecutive tiles, which read each key once
  // for the whole group. Each kind costliest first, so long items start
  // early; the two kinds in alternating runs of 256 (kRun), so that the
  // first blocks the device places, one a CU and then a second on each
  // CU, pair an arithmetic-bound group with an HBM-bound one-tile item.
  std::vector<asv_work> work;
  for (int32_t ti = 0; ti < static_cast<int32_t>(tiles.size());) {
    const asv_tile& t = tiles[ti];
    const asv_seg& g = segs[t.stream];
    const int32_t stream_tiles = (g.rows + ASV_TILE_ROWS - 1) / ASV_TILE_ROWS;
    const int32_t left = stream_tiles - t.pos0 / ASV_TILE_ROWS;
    const int32_t nt = stream_tiles == 1 ? 1 : std::min(kGroupTiles, left);
    const asv_tile& tl = tiles[ti + nt - 1];
    const int32_t n_last = full ? g.keys : g.keys - g.rows + tl.pos0 + tl.nrows;
    const Plan pl{g.split_keys, g.split_tail, g.nbig, g.nsplit};
    for (int32_t sp = 0; sp < g.nsplit && split_start(pl, sp) < n_last; ++sp) {
      const int32_t k0 = split_start(pl, sp);
      const int32_t k1 = std::min(sp + 1 < g.nsplit ? split_start(pl, sp + 1) : g.keys, n_last);
      for (int32_t h = 0; h < ASV_KV_HEADS; ++h)
        work.push_back({ti, int8_t(h), int8_t(nt), int16_t(t.stream), sp, k1 - k0});
    }
    ti += nt;
  }
  auto cost = [](const asv_work& w) { return int64_t(w.keys) * (w.ntiles > 1 ? 4 : 1); };
  std::stable_sort(work.begin(), work.end(),
                   [&](const asv_work& a, const asv_work& b) { return cost(a) > cost(b); });
  {
    std::vector<asv_work> grp, one;
    for (const asv_work& x : work) (x.ntiles > 1 ? grp : one).push_back(x);
    work.clear();
    size_t i = 0, j = 0;
    while (i < grp.size() || j < one.size()) {
      for (size_t k = 0; k < kRun && i < grp.size(); ++k) work.push_back(grp[i++]);
      for (size_t k = 0; k < kRun && j < one.size(); ++k) work.push_back(one[j++]);
    }
  }

  // ---- blob layout
  asv_table_info in;
  std::memset(&in, 0, sizeof(in));
  in.abi_version = ASV_ABI_VERSION;
  in.n_streams = S;
  in.n_rows = R;
  in.n_tiles = static_cast<int32_t>(tiles.size());
  in.n_work = static_cast<int32_t>(work.size());
  in.n_conv_layers = n_conv_layers;
  in.n_attn_layers = n_attn_layers;
  in.max_tile_rows = max_tile_rows;
  in.partial_count = poff;
  int64_t off = 0;
  in.off_segs = off;       off = align16(off + int64_t(sizeof(asv_seg)) * S);
  in.off_rows = off;       off = align16(off + int64_t(sizeof(asv_row)) * R);
  in.off_tiles = off;      off = align16(off + int64_t(sizeof(asv_tile)) * in.n_tiles);
  in.off_work = off;       off = align16(off + int64_t(sizeof(asv_work)) * in.n_work);
  in.off_conv_state = off; off = align16(off + 8 * int64_t(n_conv_layers) * S);
  in.off_k = off;          off = align16(off + 8 * int64_t(n_attn_layers) * S);
  in.off_v = off;          off = align16(off + 8 * int64_t(n_attn_layers) * S);
  in.blob_bytes = off;
  *info = in;

  if (blob == nullptr) return ASV_OK;
  if (blob_bytes < static_cast<size_t>(in.blob_bytes)) return ASV_E_CAPACITY;

  char* b = static_cast<char*>(blob);
  std::memset(b, 0, static_cast<size_t>(in.blob_bytes));
  std::memcpy(b + in.off_segs, segs.data(), sizeof(asv_seg) * S);
  std::memcpy(b + in.off_rows, rows.data(), sizeof(asv_row) * R);
  std::memcpy(b + in.off_tiles, tiles.data(), sizeof(asv_tile) * tiles.size());
  if (!work.empty()) std::memcpy(b + in.off_work, work.data(), sizeof(asv_work) * work.size());
  uint64_t* cs = reinterpret_cast<uint64_t*>(b + in.off_conv_state);
  for (int64_t i = 0; i < int64_t(n_conv_layers) * S; ++i)
    cs[i] = reinterpret_cast<uintptr_t>(conv_state[i]);
  uint64_t* kp = reinterpret_cast<uint64_t*>(b + in.off_k);
  uint64_t* vp = reinterpret_cast<uint64_t*>(b + in.off_v);
  for (int64_t i = 0; i < int64_t(n_attn_layers) * S; ++i) {
    kp[i] = reinterpret_cast<uintptr_t>(k_cache[i]);
    vp[i] = reinterpret_cast<uintptr_t>(v_cache[i]);
  }
  return ASV_OK;
}

}  // namespace

extern "C" int asv_seg_table_build(const asv_stream_desc* streams, int32_t n_streams,
                                   const void* const* conv_state, int32_t n_conv_layers,
                                   const void* const* k_cache, const void* const* v_cache,
                                   int32_t n_attn_layers, void* blob, size_t blob_bytes,
                                   asv_table_info* info) {
  return build_table(streams, n_streams, conv_state, n_conv_layers, k_cache, v_cache,
                     n_attn_layers, blob, blob_bytes, info, false);
}

extern "C" int asv_block_table_build(const asv_stream_desc* streams, int32_t n_streams,
                                     const void* const* conv_state, int32_t n_conv_layers,
                                     const void* const* k_cache, const void* const* v_cache,
                                     int32_t n_attn_layers, void* blob, size_t blob_bytes,
                                     asv_table_info* info) {
  return build_table(streams, n_streams, conv_state, n_conv_layers, k_cache, v_cache,
                     n_attn_layers, blob, blob_bytes, info, true);
}
