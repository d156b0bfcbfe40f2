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

// Merge: one wave per (row, q head); lane d owns output dim d. Lanes first
// run over the row's splits (lane j holds split t0 + j of a 64-split chunk)
// to take M = max_t m_t, then compute each split's weight
// w_t = e^(m_t - M) l_t in the lane that loaded it. A sequential pass in
// split order, t = 0, 1, ..., then adds w_t (broadcast from its lane) to L
// and w_t o_t[d] to the output; the o loads of successive splits are
// independent, so they are in flight together. Empty splits (l = 0) take
// no part; a NaN partial propagates.
constexpr int kMergeWaves = 4;

__device__ __forceinline__ float wave_max(float x) {
  x = max_xor32(max_xor16(x));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 16));
  return x;
}

__global__ __launch_bounds__(64 * kMergeWaves) void merge_rows(TableView tv,
                                                               const float* __restrict__ po,
                                                               const float* __restrict__ pml,
                                                               uint16_t* __restrict__ O) {
  const int pair = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (pair >= tv.n_rows * ASV_Q_HEADS) return;
  const int lane = threadIdx.x & 63;
  const int r = pair / ASV_Q_HEADS;
  const int h = pair - r * ASV_Q_HEADS;
  const asv_row row = uniform(cload(tv.rows + r));
  const asv_seg S = uniform(cload(tv.segs + row.stream));
  const int nt = splits_before(S, row.nkeys);
  const int64_t rec0 = S.poff + int64_t(row.pos) * ASV_Q_HEADS + h;
  const int64_t step = int64_t(S.rows) * ASV_Q_HEADS;
  const float2* ml = reinterpret_cast<const float2*>(pml);
  const float ninf = -__builtin_inff();

  // (m, l) of split t0 + lane; most rows have at most 64 splits, so the
  // first chunk's values are kept for the second pass
  float2 v0 = make_float2(ninf, 0.f);
  if (lane < nt) v0 = gload(ml + rec0 + lane * step);
  float M = (v0.y != 0.f) ? v0.x : ninf;
  for (int t = 64 + lane; t < nt; t += 64) {
    const float2 v = gload(ml + rec0 + t * step);
    if (v.y != 0.f) M = fmaxf(M, v.x);
  }
  M = wave_max(M);

  float L = 0.f, acc = 0.f;
  const float* o = po + rec0 * ASV_HEAD_DIM + lane;
  const int64_t ostep = step * ASV_HEAD_DIM;
  for (int t0 = 0; t0 < nt; t0 += 64) {
    const float2 v = (t0 == 0) ? v0 : ((t0 + lane < nt) ? gload(ml + rec0 + (t0 + lane) * step)
                                                          : make_float2(ninf, 0.f));
    const float w = exp2_((v.x - M) * kLog2e) * v.y;
    const uint64_t empty = __ballot(v.y == 0.f);
    const int n = min(64, nt - t0);
    int j0 = 0;
    for (; j0 + 8 <= n; j0 += 8) {
      // eight splits at a time, their loads in flight together
      float ot[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) ot[k] = gload(o + (t0 + j0 + k) * ostep);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = j0 + k;
        const bool use = !((empty >> j) & 1u);
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
        L = use ? L + wj : L;
        acc = use ? __builtin_fmaf(wj, ot[k], acc) : acc;
      }
    }
    for (int j = j0; j < n; ++j) {  // the rest, one split at a time
      const float ot = gload(o + (t0 + j) * ostep);
      const bool use = !((empty >> j) & 1u);
      const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
      L = use ? L + wj : L;
      acc = use ? __builtin_fmaf(wj, ot, acc) : acc;
    }
  }
  const float y = (L != 0.f) ? acc / L : 0.f;
  gstore(O + (int64_t(r) * ASV_Q_HEADS + h) * ASV_HEAD_DIM + lane, uint16_t(f32_to_bf16(y)));
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
  const unsigned pairs = unsigned(info->n_rows) * ASV_Q_HEADS;
  hipLaunchKernelGGL(asv::merge_rows, dim3((pairs + asv::kMergeWaves - 1) / asv::kMergeWaves),
                     dim3(64 * asv::kMergeWaves), 0,
                     static_cast<hipStream_t>(stream), tv, po, pml, o);
  return hipGetLastError() == hipSuccess ? ASV_OK : ASV_E_HIP;
}
