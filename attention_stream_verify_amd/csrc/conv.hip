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
// another block. Only the blocks holding a stream's first two rows (the only
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

// bx for 8 channels of one row: bf16(B * x), exact product in fp32.
__device__ __forceinline__ void bx8(const uint16_t* xrow, int c0, float out[8]) {
  const u32x4 b = load16(xrow + c0);
  const u32x4 x = load16(xrow + 2 * ASV_HIDDEN + c0);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    out[2 * k] = bf16_to_f32(uint16_t(f32_to_bf16(bf16_lo(b[k]) * bf16_lo(x[k]))));
    out[2 * k + 1] = bf16_to_f32(uint16_t(f32_to_bf16(bf16_hi(b[k]) * bf16_hi(x[k]))));
  }
}

__device__ __forceinline__ void store_bf16x8(uint16_t* p, const float v[8]) {
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = (__float_as_uint(v[2 * k]) >> 16) | (__float_as_uint(v[2 * k + 1]) & 0xFFFF0000u);
  store16(p, w);
}

__global__ __launch_bounds__(kThreads) void conv_rows(TableView tv, int layer,
                                                      const uint16_t* __restrict__ X,
                                                      const uint16_t* __restrict__ W,
                                                      uint16_t* __restrict__ Y) {
  const asv_tile T = gload(tv.tiles + blockIdx.x);
  const int i0 = blockIdx.y * kRowsPerBlock;
  if (i0 >= T.nrows) return;
  const int i1 = min(i0 + kRowsPerBlock, T.nrows);
  const asv_seg S = gload(tv.segs + T.stream);
  const int p0 = T.pos0 + i0;           // window position of the block's first row
  const int c0 = (blockIdx.z * kThreads + threadIdx.x) * 8;

  // taps of 8 channels: W[c][0..2] for c = c0..c0+7, 48 contiguous bytes
  float w0[8], w1[8], w2[8];
  {
    const u32x4 a = load16(W + c0 * 3);
    const u32x4 b = load16(W + c0 * 3 + 8);
    const u32x4 c = load16(W + c0 * 3 + 16);
    uint32_t words[12] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3], c[0], c[1], c[2], c[3]};
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

  uint16_t* state = reinterpret_cast<uint16_t*>(
      gload(tv.conv_state + int64_t(layer) * tv.n_streams + T.stream));
  float h0[8], h1[8];
  if (p0 == 0) {
    const u32x4 s0 = load16(state + c0);
    const u32x4 s1 = load16(state + ASV_HIDDEN + c0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      h0[2 * k] = bf16_lo(s0[k]);
      h0[2 * k + 1] = bf16_hi(s0[k]);
      h1[2 * k] = bf16_lo(s1[k]);
      h1[2 * k + 1] = bf16_hi(s1[k]);
    }
  } else {
    // p0 >= 2: the two history steps before the block are bx of rows p0-2, p0-1
    bx8(X + int64_t(S.row0 + p0 - 2) * ASV_CONV_IN, c0, h0);
    bx8(X + int64_t(S.row0 + p0 - 1) * ASV_CONV_IN, c0, h1);
  }

  for (int i = i0; i < i1; ++i) {
    const int64_t r = T.row0 + i;
    const uint16_t* xr = X + r * ASV_CONV_IN;
    const u32x4 cw = load16(xr + ASV_HIDDEN + c0);
    float bx[8];
    bx8(xr, c0, bx);
    float y[8];
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
      const float gate = (ch & 1) ? bf16_hi(cw[ch >> 1]) : bf16_lo(cw[ch >> 1]);
      float acc = w0[ch] * h0[ch];
      acc = __builtin_fmaf(w1[ch], h1[ch], acc);
      acc = __builtin_fmaf(w2[ch], bx[ch], acc);
      y[ch] = __uint_as_float(f32_to_bf16(gate * acc) << 16);
      h0[ch] = h1[ch];
      h1[ch] = bx[ch];
    }
    store_bf16x8(Y + r * ASV_HIDDEN + c0, y);
  }

  if (p0 == 0) {
    // new state = the last two history steps [h_w, h_{w+1}]
    if (T.pos0 + i1 != S.rows) {
      bx8(X + int64_t(S.row0 + S.rows - 2) * ASV_CONV_IN, c0, h0);
      bx8(X + int64_t(S.row0 + S.rows - 1) * ASV_CONV_IN, c0, h1);
    }
    store_bf16x8(state + c0, h0);
    store_bf16x8(state + ASV_HIDDEN + c0, h1);
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
  hipLaunchKernelGGL(asv::conv_rows, dim3(unsigned(info->n_tiles), pairs, asv::kChannelGroups),
                     dim3(asv::kThreads),
                     0, static_cast<hipStream_t>(stream), tv, int(layer), x, w, y);
  return hipGetLastError() == hipSuccess ? ASV_OK : ASV_E_HIP;
}
