// Merge of each row's split-K attention partials into the bf16 output
// (gfx950).
//
// PR #1377 "LFM2: shared-round decode", shared-round commit: the attention
// launch of a layer leaves each stream's split partials apart; one merge
// launch a layer combines every row's splits. The arithmetic per row and
// head is written out in include/asv.h.

#include "device.h"

namespace asv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge: one wave per (row, group of 4 q heads); the 16 lanes 16j..16j+15
// serve head 4g + j, lane 16j + c output dims 4c..4c+3, so each split's o
// records of the four heads (1 KB, contiguous) come in one 16-byte load a
// lane. First each head's lanes take M = max_t m_t over its non-empty
// splits (lane c looks at splits c, c + 16, ...; a max over the 16 lanes
// follows). Then one pass in split order, t = 0, 1, ..., adds
// w_t = e^(m_t - M) l_t to L and w_t o_t[d] to the output, each lane
// computing w_t from its head's (m_t, l_t) (the same 8 bytes for the 16
// lanes); the loads of 8 successive splits are in flight together. Empty
// splits (l = 0) take no part; a NaN partial propagates. The arithmetic of
// every output element, and its order, is that of one lane per element.
constexpr int kMergeWaves = 4;
constexpr int kHeadsPerWave = 4;

// Max over the 16 lanes of a row of the wave (DPP within rows).
__device__ __forceinline__ float row16_max(float x) {
  auto dmax = [](float v, int ctrl_v) { return fmaxf(v, __int_as_float(ctrl_v)); };
  x = dmax(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // ^1
  x = dmax(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // ^2
  x = dmax(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)); // 7-i
  x = dmax(x, __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)); // 15-i
  return x;
}

__global__ __launch_bounds__(64 * kMergeWaves) void merge_rows(TableView tv,
                                                               const float* __restrict__ po,
                                                               const float* __restrict__ pml,
                                                               uint16_t* __restrict__ O) {
  constexpr int kGroups = ASV_Q_HEADS / kHeadsPerWave;
  const int item = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (item >= tv.n_rows * kGroups) return;
  const int lane = threadIdx.x & 63;
  const int r = item / kGroups;
  const int h = (item - r * kGroups) * kHeadsPerWave + (lane >> 4);
  const int c = lane & 15;
  const asv_row row = uniform(cload(tv.rows + r));
  const asv_seg S = uniform(cload(tv.segs + row.stream));
  const int nt = splits_before(S, row.nkeys);
  const int64_t rec0 = S.poff + int64_t(row.pos) * ASV_Q_HEADS + h;
  const int64_t step = int64_t(S.rows) * ASV_Q_HEADS;
  const float2* ml = reinterpret_cast<const float2*>(pml);
  const float ninf = -__builtin_inff();

  float M = ninf;
  for (int t = c; t < nt; t += 16) {
    const float2 v = gload(ml + rec0 + t * step);
    if (v.y != 0.f) M = fmaxf(M, v.x);
  }
  M = row16_max(M);

  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const float* o = po + rec0 * ASV_HEAD_DIM + 4 * c;
  const int64_t ostep = step * ASV_HEAD_DIM;
  auto add = [&](const float2 v, const f32x4 ot) {
    const float w = exp2_((v.x - M) * kLog2e) * v.y;
    const bool use = v.y != 0.f;
    L = use ? L + w : L;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = use ? __builtin_fmaf(w, ot[e], acc[e]) : acc[e];
  };
  int t = 0;
  for (; t + 8 <= nt; t += 8) {
    // eight splits at a time, their loads in flight together
    float2 v[8];
    f32x4 ot[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[k] = gload(ml + rec0 + (t + k) * step);
      ot[k] = gload(reinterpret_cast<const f32x4*>(o + (t + k) * ostep));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) add(v[k], ot[k]);
  }
  for (; t < nt; ++t)  // the rest, one split at a time
    add(gload(ml + rec0 + t * step), gload(reinterpret_cast<const f32x4*>(o + t * ostep)));
  uint32_t y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = f32_to_bf16((L != 0.f) ? acc[e] / L : 0.f);
  gstore(reinterpret_cast<unsigned long long*>(O + (int64_t(r) * ASV_Q_HEADS + h) * ASV_HEAD_DIM +
                                               4 * c),
         (unsigned long long)(y[0] | (y[1] << 16)) |
             ((unsigned long long)(y[2] | (y[3] << 16)) << 32));
}

}  // namespace
}  // namespace asv

extern "C" int asv_attn_merge(const asv_table_info* info, const void* dev_blob,
                              const float* partials, uint16_t* o, void* stream) {
  if (!asv::info_ok(info) || dev_blob == nullptr || partials == nullptr || o == nullptr)
    return ASV_E_ARG;
  if (!asv::aligned16(dev_blob) || !asv::aligned16(partials) || !asv::aligned16(o))
    return ASV_E_ARG;
  const asv::TableView tv = asv::make_view(*info, dev_blob);
  const float* po = partials;
  const float* pml = partials + info->partial_count * ASV_HEAD_DIM;
  const unsigned items = unsigned(info->n_rows) * (ASV_Q_HEADS / asv::kHeadsPerWave);
  hipLaunchKernelGGL(asv::merge_rows, dim3((items + asv::kMergeWaves - 1) / asv::kMergeWaves),
                     dim3(64 * asv::kMergeWaves), 0,
                     static_cast<hipStream_t>(stream), tv, po, pml, o);
  return hipGetLastError() == hipSuccess ? ASV_OK : ASV_E_HIP;
}
