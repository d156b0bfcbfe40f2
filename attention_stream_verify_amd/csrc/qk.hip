// qk stage of an attention layer over every row of a shared round (gfx950):
// q and k head RMS norm, half-split RoPE, and the K/V append into every
// stream's cache through the table.
//
// PR #1377 "LFM2: shared-round decode": an attention layer is a qk launch,
// the attention and the merge, and the shared round runs each once a layer
// over every row through the table of cache addresses, row offsets and key
// counts. PR #1391 (the DSpark drafter): the target's RoPE kernel is
// half-split and the q and k rows carry norm gains. The arithmetic is
// written out in include/asv_qk.h.
//
// Mapping: one block of 384 threads a row; each thread owns 8 consecutive
// values of the row's 3,072 (one 16-byte load, 1 KB a wave): threads 0-255
// are the 32 q heads, 256-319 the 8 k heads, 320-383 (the sixth wave) the 8
// v heads. A head is 8 consecutive lanes, so its sum of squares is three
// butterflies and the RoPE partner of values 0-31 (lanes 0-3 of the head)
// is the lane 4 away. The 32 (cos, sin) pairs of the row's position are
// formed once per block in float64 (angle, reduction to [-pi, pi], then the
// float64 sine and cosine), so large positions keep their accuracy.

#include <cmath>

#include "device.h"
#include "asv_qk.h"

namespace asv {
namespace {

constexpr int kThreads = ASV_QKV_WIDTH / 8;   // 384
constexpr int kQLanes = ASV_Q_HEADS * 8;      // 256
constexpr int kKLanes = ASV_KV_HEADS * 8;     // 64

__device__ __forceinline__ float xor_sum8(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x;
}

__global__ __launch_bounds__(kThreads) void qk_rows(TableView tv, int layer, const uint16_t* __restrict__ qkv,
                                                    const uint16_t* __restrict__ q_gain,
                                                    const uint16_t* __restrict__ k_gain, double log2_theta,
                                                    float eps, uint16_t* __restrict__ q_out) {
  __shared__ float s_cos[ASV_HEAD_DIM / 2];
  __shared__ float s_sin[ASV_HEAD_DIM / 2];
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const asv_row R = uniform(gload(tv.rows + r));
  const asv_seg S = uniform(gload(tv.segs + R.stream));
  const int pos = S.keys - S.rows + R.pos;
  if (t < ASV_HEAD_DIM / 2) {
    const double a = double(pos) * exp2(-double(t) / double(ASV_HEAD_DIM / 2) * log2_theta);
    const double two_pi = 6.283185307179586476925286766559;
    const double red = a - two_pi * rint(a / two_pi);
    s_cos[t] = float(cos(red));
    s_sin[t] = float(sin(red));
  }
  const u32x4 x = load16(qkv + int64_t(r) * ASV_QKV_WIDTH + t * 8);
  __syncthreads();

  const int64_t sel = int64_t(layer) * tv.n_streams + R.stream;
  const int sub = t & 7;   // values 8*sub .. 8*sub+7 of the head
  if (t >= kQLanes + kKLanes) {
    // v: copied into the d-major 32-key block of key pos
    const int h = (t - kQLanes - kKLanes) >> 3;
    uint16_t* vc = reinterpret_cast<uint16_t*>(uniform_ptr(cload(tv.vp + sel)));
    uint16_t* blk = vc + ((int64_t(h) * (S.cap / ASV_KEY_BLOCK) + pos / ASV_KEY_BLOCK) * ASV_HEAD_DIM) *
                             ASV_KEY_BLOCK + pos % ASV_KEY_BLOCK;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint16_t b = uint16_t((j & 1) ? (x[j >> 1] >> 16) : (x[j >> 1] & 0xFFFFu));
      gstore(blk + int64_t(sub * 8 + j) * ASV_KEY_BLOCK, b);
    }
    return;
  }

  const bool is_q = t < kQLanes;
  const u32x4 gw = load16((is_q ? q_gain : k_gain) + sub * 8);
  float f[8], g[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[2 * k] = bf16_lo(x[k]);
    f[2 * k + 1] = bf16_hi(x[k]);
    g[2 * k] = bf16_lo(gw[k]);
    g[2 * k + 1] = bf16_hi(gw[k]);
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss = __builtin_fmaf(f[j], f[j], ss);
  ss = xor_sum8(ss);
  const float inv = 1.0f / sqrtf(ss * (1.0f / ASV_HEAD_DIM) + eps);
  float y[8], p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = f[j] * inv * g[j];
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = __shfl_xor(y[j], 4);
  const bool lo = sub < 4;   // values 0..31: out = y c - partner s; 32..63: y c + partner s
  const int i0 = (sub & 3) * 8;
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float o[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = 2 * k + e;
      const float c = s_cos[i0 + j], s = s_sin[i0 + j];
      o[e] = lo ? y[j] * c - p[j] * s : y[j] * c + p[j] * s;
    }
    w[k] = pack_bf16x2(o[0], o[1]);
  }
  u32x4 out;
  out[0] = w[0];
  out[1] = w[1];
  out[2] = w[2];
  out[3] = w[3];
  if (is_q) {
    store16(q_out + int64_t(r) * (ASV_Q_HEADS * ASV_HEAD_DIM) + t * 8, out);
  } else {
    const int h = (t - kQLanes) >> 3;
    uint16_t* kc = reinterpret_cast<uint16_t*>(uniform_ptr(cload(tv.kp + sel)));
    store16(kc + (int64_t(h) * S.cap + pos) * ASV_HEAD_DIM + sub * 8, out);
  }
}

}  // namespace
}  // namespace asv

extern "C" int asv_shared_qk(const asv_table_info* info, const void* dev_blob, int32_t layer,
                             const uint16_t* qkv, const uint16_t* q_gain, const uint16_t* k_gain, double theta,
                             double eps, uint16_t* q_out, void* stream) {
  if (!asv::info_ok(info) || dev_blob == nullptr || qkv == nullptr || q_gain == nullptr ||
      k_gain == nullptr || q_out == nullptr)
    return ASV_E_ARG;
  if (!asv::aligned16(dev_blob) || !asv::aligned16(qkv) || !asv::aligned16(q_gain) ||
      !asv::aligned16(k_gain) || !asv::aligned16(q_out))
    return ASV_E_ARG;
  const char* a = reinterpret_cast<const char*>(qkv);
  const char* b = reinterpret_cast<const char*>(q_out);
  const int64_t R = info->n_rows;
  if (a < b + R * ASV_Q_HEADS * ASV_HEAD_DIM * 2 && b < a + R * ASV_QKV_WIDTH * 2) return ASV_E_ARG;
  if (layer < 0 || layer >= info->n_attn_layers) return ASV_E_SHAPE;
  if (!std::isfinite(theta) || !(theta > 0.0) || !std::isfinite(eps) || !(eps >= 0.0)) return ASV_E_SHAPE;
  const asv::TableView tv = asv::make_view(*info, dev_blob);
  hipLaunchKernelGGL(asv::qk_rows, dim3(unsigned(R)), dim3(asv::kThreads), 0, static_cast<hipStream_t>(stream), tv,
                     int(layer), qkv, q_gain, k_gain, std::log2(theta), float(eps), q_out);
  return hipGetLastError() == hipSuccess ? ASV_OK : ASV_E_HIP;
}
