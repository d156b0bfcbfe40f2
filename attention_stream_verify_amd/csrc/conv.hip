// Gated short conv of one layer over every row of a shared round (gfx950).
//
// PR #1377 "LFM2: shared-round decode", shared-round commit: one conv launch
// a layer over the rows of every stream, each row against its own stream's
// conv state (the pages count 30 conv layers a forward). The arithmetic per
// row is written out in include/asv.h: B|C|x from the 6,144-wide input,
// bx = bf16(B*x), three causal taps over [state, bx...], gate C, and the
// state advanced to the last two steps.
//
// Mapping: a 64-thread block covers 2 rows of one 16-row tile and 512 of the
// 2,048 channels; each thread owns 8 channels (16-byte loads of B, C, x: one
// block reads 1 KB contiguous per input third). Small rounds are latency
// bound, so the grid is made wide (tiles x row pairs x 4 channel groups,
// the row pairs of the round's largest tile) rather than deep. Rows are
// independent once bx of the two rows before them
// is known, so a block recomputes those from X instead of waiting for
// another block. A block issues all of its loads (rows, taps, history, and
// the rows the new state needs) as soon as its tile record is read, so it
// waits for memory once. Only the blocks holding a stream's first two rows (the only
// rows that read the state) touch the stream's state: each reads its
// channels of the state, then writes them anew, so no thread ever reads a
// state that another thread is rewriting.

#include "device.h"

namespace asv {
namespace {

constexpr int kThreads = 64;    // 8 channels each -> 512 a block
constexpr int kChannelGroups = ASV_HIDDEN / (kThreads * 8);
constexpr int kRowsPerBlock = 2;
constexpr int kSub = ASV_TILE_ROWS / kRowsPerBlock;

// bx for 8 channels of one row from its loaded B and x words: bf16(B * x),
// the exact product in fp32 rounded once.
__device__ __forceinline__ void bx8(const u32x4& b, const u32x4& x, float out[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    out[2 * k] = bf16_to_f32(uint16_t(f32_to_bf16(bf16_lo(b[k]) * bf16_lo(x[k]))));
    out[2 * k + 1] = bf16_to_f32(uint16_t(f32_to_bf16(bf16_hi(b[k]) * bf16_hi(x[k]))));
  }
}

__device__ __forceinline__ void words8(const u32x4& w, float out[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    out[2 * k] = bf16_lo(w[k]);
    out[2 * k + 1] = bf16_hi(w[k]);
  }
}

__device__ __forceinline__ void store_bf16x8(uint16_t* p, const float v[8]) {
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = (__float_as_uint(v[2 * k]) >> 16) | (__float_as_uint(v[2 * k + 1]) & 0xFFFF0000u);
  store16(p, w);
}

// One row: y = C * (w0 h0 + w1 h1 + w2 bx) for 8 channels, then the history
// moves on by one step.
__device__ __forceinline__ void conv_row(const u32x4& b, const u32x4& c, const u32x4& x, const float w0[8],
                                         const float w1[8], const float w2[8], float h0[8], float h1[8],
                                         uint16_t* yrow) {
  float bx[8];
  bx8(b, x, bx);
  float y[8];
#pragma unroll
  for (int ch = 0; ch < 8; ++ch) {
    const float gate = (ch & 1) ? bf16_hi(c[ch >> 1]) : bf16_lo(c[ch >> 1]);
    float acc = w0[ch] * h0[ch];
    acc = __builtin_fmaf(w1[ch], h1[ch], acc);
    acc = __builtin_fmaf(w2[ch], bx[ch], acc);
    y[ch] = __uint_as_float(f32_to_bf16(gate * acc) << 16);
    h0[ch] = h1[ch];
    h1[ch] = bx[ch];
  }
  store_bf16x8(yrow, y);
}

// Block order on the device: blocks are dealt to the 8 XCDs in turn (the
// grid's linear index mod 8, each XCD with its own L2). With several row
// pairs a tile the grid is (8, pairs, tiles8 / 2), tiles8 = the tile count
// rounded up to 8: a block's XCD is blockIdx.x, and the row pairs of a
// group g = blockIdx.x + 8 blockIdx.z = tile * 4 + channel group share it. A
// row pair reads as history the two rows the pair before it reads as its
// own, and on one XCD those rows leave HBM once (at 2,048 rows the launch
// fetched 1.70x its input bytes when they did not, 1.09x now); blocks past
// the last tile exit. With one pair (one-row windows) the grid is (tiles, 1,
// 4): a tile's four channel groups land on one XCD, with its table records.
template <bool ONE_PAIR>
__device__ __forceinline__ void conv_block(int& tile, int& cgroup, int& pair) {
  if (ONE_PAIR) {
    tile = int(blockIdx.x);
    cgroup = int(blockIdx.z);
    pair = 0;
  } else {
    const int g = int(blockIdx.x) + 8 * int(blockIdx.z);
    tile = g >> 2;
    cgroup = g & 3;
    pair = int(blockIdx.y);
  }
}

template <bool ONE_PAIR>
__global__ __launch_bounds__(kThreads) void conv_rows(TableView tv, int layer,
                                                      const uint16_t* __restrict__ X,
                                                      const uint16_t* __restrict__ W,
                                                      uint16_t* __restrict__ Y) {
  static_assert(kRowsPerBlock == 2, "a block holds one or two rows");
  // The launch arguments the block uses, read into scalar registers together
  // with the tile pointer (otherwise each is read where first used, after
  // the early exit below, one round trip after another).
  const asv_seg* segs = tv.segs;
  const uint64_t* cstate = tv.conv_state;
  const int nstreams = tv.n_streams;
  asm volatile("" ::"s"(segs), "s"(cstate), "s"(nstreams), "s"(layer), "s"(X), "s"(W), "s"(Y));
  int tile, cgroup, pair;
  conv_block<ONE_PAIR>(tile, cgroup, pair);
  if (!ONE_PAIR && tile >= tv.n_tiles) return;  // padding past the last tile
  const asv_tile T = cload(tv.tiles + tile);
  const int i0 = pair * kRowsPerBlock;
  if (i0 >= T.nrows) return;
  const bool two = i0 + 1 < T.nrows;
  const int p0 = T.pos0 + i0;           // window position of the block's first row (even)
  const int c0 = (cgroup * kThreads + threadIdx.x) * 8;
  const int64_t r0 = int64_t(T.row0) + i0;

  // Every load of the block is issued before any is waited for, so the
  // block pays one memory round trip: its rows' B, C, x (a missing second
  // row re-reads the first), the taps, and the history: bx of the two rows
  // before the block (rows r0 - 2, r0 - 1 of the same stream when p0 >= 2),
  // or, for a stream's first rows, its state and, when the stream has rows
  // past the block, its last two rows for the new state. The history
  // addresses are selected rather than branched on; a load a block does
  // not need re-reads an address it reads anyway.
  const uint16_t* xa = X + r0 * ASV_CONV_IN;
  const uint16_t* xb = xa + (two ? ASV_CONV_IN : 0);
  const bool first = p0 == 0;
  // The stream's row0 and rows and its state pointer in one round trip:
  // the values pass through one asm, so nothing computed from either moves
  // ahead of the other's read. Only the record's first 8 bytes are read: a
  // 16-byte read leaves two dead words whose registers the compiler reuses
  // for the pointer's address, waiting for the record first.
  static_assert(offsetof(asv_seg, row0) == 0 && offsetof(asv_seg, rows) == 4, "asv_seg layout");
  const uint64_t rr = cload(reinterpret_cast<const uint64_t*>(segs + T.stream));
  uint16_t* state = reinterpret_cast<uint16_t*>(cload(cstate + int64_t(layer) * nstreams + T.stream));
  int srow0 = int(uint32_t(rr)), srows = int(uint32_t(rr >> 32));
  asm volatile("" : "+s"(state), "+s"(srow0), "+s"(srows));
  const bool tail = first && (two ? 2 : 1) != srows;
  const u32x4 ba = load16(xa + c0), ca = load16(xa + ASV_HIDDEN + c0), xa2 = load16(xa + 2 * ASV_HIDDEN + c0);
  const u32x4 bb = load16(xb + c0), cb = load16(xb + ASV_HIDDEN + c0), xb2 = load16(xb + 2 * ASV_HIDDEN + c0);
  const u32x4 wa = load16(W + c0 * 3), wb = load16(W + c0 * 3 + 8), wc = load16(W + c0 * 3 + 16);
  // History: p0 >= 2, B and x of rows r0 - 2 and r0 - 1; p0 == 0, the
  // state's two steps (hb0, hb1; hx0 and hx1 re-read them). Each selected
  // address passes through an empty asm, so the compiler cannot see which
  // operand it is: it would otherwise merge a re-read with the load it
  // repeats, or turn the select back into a branch.
  const uint16_t* h0 = first ? state : xa - 2 * ASV_CONV_IN;
  const uint16_t* h1 = first ? state + ASV_HIDDEN : xa - ASV_CONV_IN;
  int hx = first ? 0 : 2 * ASV_HIDDEN;
  asm("" : "+s"(h0), "+s"(h1), "+s"(hx));
  const u32x4 hb0 = load16(h0 + c0), hx0 = load16(h0 + hx + c0);
  const u32x4 hb1 = load16(h1 + c0), hx1 = load16(h1 + hx + c0);
  // B and x of the stream's last two rows when the new state needs them
  const uint16_t* xl = tail ? X + (int64_t(srow0) + srows - 2) * ASV_CONV_IN : xa;
  int ln = tail ? ASV_CONV_IN : 0;
  asm("" : "+s"(xl), "+s"(ln));
  const u32x4 lb0 = load16(xl + c0), lx0 = load16(xl + 2 * ASV_HIDDEN + c0);
  const u32x4 lb1 = load16(xl + ln + c0), lx1 = load16(xl + ln + 2 * ASV_HIDDEN + c0);
  // Compiler-only barriers: no memory access (asm) and no instruction
  // (sched_barrier) moves across them, so the loads above are all issued
  // before any of their results is waited for (neither makes the hardware
  // wait for anything).
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // taps of 8 channels: W[c][0..2] for c = c0..c0+7, 48 contiguous bytes
  float w0[8], w1[8], w2[8];
  {
    const uint32_t words[12] = {wa[0], wa[1], wa[2], wa[3], wb[0], wb[1], wb[2], wb[3], wc[0], wc[1], wc[2], wc[3]};
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int e = ch * 3 + k;
        const float v = (e & 1) ? bf16_hi(words[e >> 1]) : bf16_lo(words[e >> 1]);
        if (k == 0) w0[ch] = v;
        else if (k == 1) w1[ch] = v;
        else w2[ch] = v;
      }
    }
  }

  float g0[8], g1[8];   // the two history steps before the next row
  if (first) {
    words8(hb0, g0);
    words8(hb1, g1);
  } else {
    bx8(hb0, hx0, g0);
    bx8(hb1, hx1, g1);
  }
  conv_row(ba, ca, xa2, w0, w1, w2, g0, g1, Y + r0 * ASV_HIDDEN + c0);
  if (two) conv_row(bb, cb, xb2, w0, w1, w2, g0, g1, Y + (r0 + 1) * ASV_HIDDEN + c0);

  if (first) {
    // new state = the last two history steps [h_w, h_{w+1}]
    if (tail) {
      bx8(lb0, lx0, g0);
      bx8(lb1, lx1, g1);
    }
    store_bf16x8(state + c0, g0);
    store_bf16x8(state + ASV_HIDDEN + c0, g1);
  }
}

}  // namespace
}  // namespace asv

extern "C" int asv_shared_conv(const asv_table_info* info, const void* dev_blob, int32_t layer,
                               const uint16_t* x, const uint16_t* w, uint16_t* y, void* stream) {
  if (!asv::info_ok(info) || dev_blob == nullptr || x == nullptr || w == nullptr || y == nullptr)
    return ASV_E_ARG;
  if (!asv::aligned16(dev_blob) || !asv::aligned16(x) || !asv::aligned16(w) || !asv::aligned16(y))
    return ASV_E_ARG;
  if (layer < 0 || layer >= info->n_conv_layers) return ASV_E_SHAPE;
  const asv::TableView tv = asv::make_view(*info, dev_blob);
  // row pairs a tile: as many as the round's largest tile needs (one for
  // one-row decode windows), so no block is launched only to exit
  const unsigned pairs = unsigned((info->max_tile_rows + asv::kRowsPerBlock - 1) / asv::kRowsPerBlock);
  if (pairs < 1 || pairs > unsigned(asv::kSub)) return ASV_E_ARG;
  static_assert(asv::kChannelGroups == 4, "the block order assumes four channel groups");
  const unsigned tiles8 = (unsigned(info->n_tiles) + 7) / 8 * 8;
  if (pairs == 1)
    hipLaunchKernelGGL(asv::conv_rows<true>, dim3(unsigned(info->n_tiles), 1, asv::kChannelGroups),
                       dim3(asv::kThreads), 0, static_cast<hipStream_t>(stream), tv, int(layer), x, w, y);
  else
    hipLaunchKernelGGL(asv::conv_rows<false>, dim3(8, pairs, tiles8 / 2), dim3(asv::kThreads), 0,
                       static_cast<hipStream_t>(stream), tv, int(layer), x, w, y);
  return hipGetLastError() == hipSuccess ? ASV_OK : ASV_E_HIP;
}
