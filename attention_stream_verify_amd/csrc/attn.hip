// Split-K GQA attention over every stream of a shared round, and the merge
// of each row's split partials (gfx950).
//
// PR #1377 "LFM2: shared-round decode", shared-round commit: one attention
// launch a layer covers every stream's rows through the segment table; each
// stream's partials are held apart in the scratch; one merge launch follows.
// The per-record arithmetic is written out in include/asv.h.
//
// Work item = (16-row tile, kv head, split). One 256-thread block per item;
// its 4 wave64s take the split's 32-key blocks in turn (wave w: blocks w,
// w+4, ...), each keeping its own online softmax, and fold their states
// through LDS in wave order at the end. A tile's q rows are its rows x the 4
// q heads of the kv head: up to 64 q vectors, in NQT = ceil(rows/4) MFMA
// column tiles of 16.
//
// Per 32-key block, on the bf16 16x16x32 MFMA (fp32 accumulate):
//   S^T[key][q]  = K[key][:] . Q[q][:]        (2 key tiles x NQT x 2 d-steps)
//   O^T[d][q]   += V^T[d][key] P^T[key][q]    (4 d tiles x NQT, P split hi+lo)
// Every operand is one 16-byte global load straight into registers: K rows
// are key-major, and V is stored d-major inside 32-key blocks, so the PV
// operand (8 consecutive keys of one d) is contiguous too. No LDS staging or
// transposition sits on the K/V stream.
//
// Lane l (G = l/16, c = l%16) of a score tile holds keys 8G+i (first tile)
// and 8G+4+i (second tile), i = 0..3, for q column c: the key rows the two
// tiles load are arranged so that these 8 keys are exactly the ones the lane
// must supply as the P operand of the PV MFMA, and the V operand of the same
// lane is V^T[d][8G..8G+7]. P is fed as two bf16 parts (hi = the top 16 bits
// of the fp32 weight, lo = the rest) so the partials keep ~16 bits of the
// weights, not bf16's 8.
//
// Bits depend only on the item's own stream: the split plan comes from the
// stream's rows and keys, each item writes its own records, and the fold
// order is fixed, so a shared round gives the same bits as each stream run
// alone.

#include "device.h"

namespace asv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kScale = 0.125f;            // 1/sqrt(64)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// Key (within a 32-key block) that MFMA row m of score tile `t` (0 or 1) holds.
__device__ __forceinline__ int key_row(int m, int t) { return 8 * (m >> 2) + 4 * t + (m & 3); }

__device__ __forceinline__ uint32_t zero_past(uint32_t w, int key, int keys) {
  if (key >= keys) w &= 0xFFFF0000u;
  if (key + 1 >= keys) w &= 0x0000FFFFu;
  return w;
}

struct KV {
  u32x4 ka0, ka1, kb0, kb1;  // K operands: tile 0/1 x d-step 0/1
  u32x4 v[4];                // V^T operands: d tiles 0..3
};

__device__ __forceinline__ void load_kv(KV& o, const uint16_t* __restrict__ Kh,
                                        const uint16_t* __restrict__ Vh, int kb, int G, int c16) {
  const uint16_t* ka = Kh + int64_t(kb + key_row(c16, 0)) * ASV_HEAD_DIM + 8 * G;
  const uint16_t* kk = Kh + int64_t(kb + key_row(c16, 1)) * ASV_HEAD_DIM + 8 * G;
  o.ka0 = load16(ka);
  o.ka1 = load16(ka + 32);
  o.kb0 = load16(kk);
  o.kb1 = load16(kk + 32);
  const uint16_t* vb = Vh + int64_t(kb >> 5) * (ASV_HEAD_DIM * 32) + c16 * 32 + 8 * G;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o.v[dt] = load16(vb + dt * 16 * 32);
}

template <int NQT>
__device__ __forceinline__ void attn_item(const TableView& tv, int layer,
                                          const uint16_t* __restrict__ Q, float* __restrict__ po,
                                          float* __restrict__ pml, const asv_work wk,
                                          float* __restrict__ lds) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = lane >> 4;
  const int c16 = lane & 15;
  const asv_tile T = tv.tiles[wk.tile];
  const asv_seg S = tv.segs[T.stream];
  const int g = wk.head;
  const int base_n = S.keys - S.rows + T.pos0;  // tile row i sees base_n + i + 1 keys
  const int n_first = base_n + 1;
  const int k0 = wk.split * S.split_keys;
  const int k1 = min(k0 + S.split_keys, base_n + T.nrows);
  const int64_t head_elems = int64_t(S.cap) * ASV_HEAD_DIM;
  const int64_t sel = int64_t(layer) * tv.n_streams + T.stream;
  const uint16_t* Kh = reinterpret_cast<const uint16_t*>(tv.kp[sel]) + g * head_elems;
  const uint16_t* Vh = reinterpret_cast<const uint16_t*>(tv.vp[sel]) + g * head_elems;

  // Q operands (B of the score MFMA) and each column's visible key count
  u32x4 qop[NQT][2];
  int nq[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int q = qt * 16 + c16;
    const int rt = q >> 2;
    if (rt < T.nrows) {
      const uint16_t* qp =
          Q + (int64_t(T.row0 + rt) * ASV_Q_HEADS + g * 4 + (q & 3)) * ASV_HEAD_DIM + 8 * G;
      qop[qt][0] = load16(qp);
      qop[qt][1] = load16(qp + 32);
      nq[qt] = base_n + rt + 1;
    } else {
      qop[qt][0] = u32x4{0u, 0u, 0u, 0u};
      qop[qt][1] = u32x4{0u, 0u, 0u, 0u};
      nq[qt] = 0;
    }
  }

  const float c = kScale * kLog2e;
  const float ninf = -__builtin_inff();
  f32x4 acc[4][NQT];
  float m[NQT], l[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    m[qt] = ninf;
    l[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  int kb = k0 + wave * 32;
  KV cur;
  if (kb < k1) load_kv(cur, Kh, Vh, kb, G, c16);
  for (; kb < k1; kb += kWaves * 32) {
    KV nxt;
    const int kn = kb + kWaves * 32;
    if (kn < k1) load_kv(nxt, Kh, Vh, kn, G, c16);

    if (kb + 32 > S.keys) {  // slots past the key count may hold anything
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int w = 0; w < 4; ++w) cur.v[dt][w] = zero_past(cur.v[dt][w], kb + 8 * G + 2 * w, S.keys);
    }
    const bool edge = kb + 32 > n_first;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      f32x4 sa = mfma(cur.ka0, qop[qt][0], f32x4{0.f, 0.f, 0.f, 0.f});
      sa = mfma(cur.ka1, qop[qt][1], sa);
      f32x4 sb = mfma(cur.kb0, qop[qt][0], f32x4{0.f, 0.f, 0.f, 0.f});
      sb = mfma(cur.kb1, qop[qt][1], sb);
      float s[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
      if (edge) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (kb + 8 * G + j >= nq[qt]) s[j] = ninf;
      }
      float mx = s[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, s[j]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m[qt], mx);
      const float nmc = -((mn == ninf) ? 0.f : mn) * c;
      const float alpha = exp2_(__builtin_fmaf(m[qt], c, nmc));
      m[qt] = mn;
      float p[8];
      float ls = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = exp2_(__builtin_fmaf(s[j], c, nmc));
        ls += p[j];
      }
      l[qt] = __builtin_fmaf(l[qt], alpha, ls);
      u32x4 hi, lo;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a = __float_as_uint(p[2 * w]);
        const uint32_t b = __float_as_uint(p[2 * w + 1]);
        hi[w] = (a >> 16) | (b & 0xFFFF0000u);
        const float ra = p[2 * w] - __uint_as_float(a & 0xFFFF0000u);
        const float rb = p[2 * w + 1] - __uint_as_float(b & 0xFFFF0000u);
        lo[w] = (__float_as_uint(ra) >> 16) | (__float_as_uint(rb) & 0xFFFF0000u);
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        f32x4 a = acc[dt][qt] * alpha;
        a = mfma(cur.v[dt], hi, a);
        acc[dt][qt] = mfma(cur.v[dt], lo, a);
      }
    }
    cur = nxt;
  }

  // each lane summed its own keys of a column; add the 4 lane groups
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    l[qt] += __shfl_xor(l[qt], 16);
    l[qt] += __shfl_xor(l[qt], 32);
  }

  // fold the waves' states in wave order through LDS
  constexpr int kPerWave = NQT * 64 * 18;  // m, l, then 4 x NQT f32x4 per lane
  if (wave > 0) {
    float* my = lds + (wave - 1) * kPerWave;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      my[qt * 64 + lane] = m[qt];
      my[(NQT + qt) * 64 + lane] = l[qt];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *reinterpret_cast<f32x4*>(my + 2 * NQT * 64 + ((dt * NQT + qt) * 64 + lane) * 4) = acc[dt][qt];
    }
  }
  __syncthreads();
  if (wave != 0) return;
  for (int w = 1; w < kWaves; ++w) {
    const float* o = lds + (w - 1) * kPerWave;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const float mw = o[qt * 64 + lane];
      const float lw = o[(NQT + qt) * 64 + lane];
      const float mn = fmaxf(m[qt], mw);
      const float nmc = -((mn == ninf) ? 0.f : mn) * c;
      const float a0 = exp2_(__builtin_fmaf(m[qt], c, nmc));
      const float a1 = exp2_(__builtin_fmaf(mw, c, nmc));
      m[qt] = mn;
      l[qt] = __builtin_fmaf(lw, a1, l[qt] * a0);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const f32x4 ow =
            *reinterpret_cast<const f32x4*>(o + 2 * NQT * 64 + ((dt * NQT + qt) * 64 + lane) * 4);
        f32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = __builtin_fmaf(ow[i], a1, acc[dt][qt][i] * a0);
        acc[dt][qt] = r;
      }
    }
  }

  // records: o normalised by l, then (m in score units, l)
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int q = qt * 16 + c16;
    const int rt = q >> 2;
    if (rt >= T.nrows) continue;
    const int64_t rec = S.poff + (int64_t(wk.split) * S.rows + T.pos0 + rt) * ASV_Q_HEADS + g * 4 + (q & 3);
    const float L = l[qt];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (L > 0.f) ? acc[dt][qt][i] / L : 0.f;
      *reinterpret_cast<f32x4*>(po + rec * ASV_HEAD_DIM + dt * 16 + 4 * G) = r;
    }
    if (G == 0) {
      pml[rec * 2] = (m[qt] == ninf) ? ninf : m[qt] * kScale;
      pml[rec * 2 + 1] = L;
    }
  }
}

template <int NQT_MAX>
__global__ __launch_bounds__(kThreads) void attn_split(TableView tv, int layer,
                                                       const uint16_t* __restrict__ Q,
                                                       float* __restrict__ po,
                                                       float* __restrict__ pml) {
  __shared__ __attribute__((aligned(16))) float lds[(kWaves - 1) * NQT_MAX * 64 * 18];
  const asv_work wk = tv.work[blockIdx.x];
  const int nqt = (tv.tiles[wk.tile].nrows + 3) >> 2;
  if constexpr (NQT_MAX >= 4) {
    if (nqt == 4) return attn_item<4>(tv, layer, Q, po, pml, wk, lds);
  }
  if constexpr (NQT_MAX >= 3) {
    if (nqt == 3) return attn_item<3>(tv, layer, Q, po, pml, wk, lds);
  }
  if constexpr (NQT_MAX >= 2) {
    if (nqt == 2) return attn_item<2>(tv, layer, Q, po, pml, wk, lds);
  }
  attn_item<1>(tv, layer, Q, po, pml, wk, lds);
}

// Merge: 16 threads per (row, q head), 4 output dims each.
__global__ __launch_bounds__(256) void merge_rows(TableView tv, const float* __restrict__ po,
                                                  const float* __restrict__ pml,
                                                  uint16_t* __restrict__ O) {
  const int pair = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (pair >= tv.n_rows * ASV_Q_HEADS) return;
  const int r = pair / ASV_Q_HEADS;
  const int h = pair - r * ASV_Q_HEADS;
  const int d0 = (threadIdx.x & 15) * 4;
  const asv_row row = tv.rows[r];
  const asv_seg S = tv.segs[row.stream];
  const int nt = (row.nkeys + S.split_keys - 1) / S.split_keys;
  const int64_t rec0 = S.poff + int64_t(row.pos) * ASV_Q_HEADS + h;
  const int64_t step = int64_t(S.rows) * ASV_Q_HEADS;
  const float ninf = -__builtin_inff();

  float M = ninf;
  for (int t = 0; t < nt; ++t) {
    const float2 ml = *reinterpret_cast<const float2*>(pml + (rec0 + t * step) * 2);
    if (ml.y != 0.f) M = fmaxf(M, ml.x);
  }
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < nt; ++t) {
    const int64_t rec = rec0 + t * step;
    const float2 ml = *reinterpret_cast<const float2*>(pml + rec * 2);
    if (ml.y == 0.f) continue;  // empty split; a NaN partial falls through and propagates
    const float w = exp2_((ml.x - M) * kLog2e) * ml.y;
    L += w;
    const f32x4 o = *reinterpret_cast<const f32x4*>(po + rec * ASV_HEAD_DIM + d0);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(w, o[i], acc[i]);
  }
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = (L != 0.f) ? acc[i] / L : 0.f;
  uint2 out;
  out.x = pack_bf16x2(y[0], y[1]);
  out.y = pack_bf16x2(y[2], y[3]);
  *reinterpret_cast<uint2*>(O + (int64_t(r) * ASV_Q_HEADS + h) * ASV_HEAD_DIM + d0) = out;
}

}  // namespace
}  // namespace asv

extern "C" int asv_shared_attn(const asv_table_info* info, const void* dev_blob, int32_t layer,
                               const uint16_t* q, float* partials, void* stream) {
  if (!asv::info_ok(info) || dev_blob == nullptr || q == nullptr || partials == nullptr)
    return ASV_E_ARG;
  if (!asv::aligned16(dev_blob) || !asv::aligned16(q) || !asv::aligned16(partials))
    return ASV_E_ARG;
  if (layer < 0 || layer >= info->n_attn_layers) return ASV_E_SHAPE;
  if (info->n_work < 1 || info->max_tile_rows < 1 || info->max_tile_rows > ASV_TILE_ROWS)
    return ASV_E_ARG;
  const asv::TableView tv = asv::make_view(*info, dev_blob);
  float* po = partials;
  float* pml = partials + info->partial_count * ASV_HEAD_DIM;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned(info->n_work)), block(asv::kThreads);
  switch ((info->max_tile_rows + 3) >> 2) {
    case 1: hipLaunchKernelGGL(asv::attn_split<1>, grid, block, 0, st, tv, int(layer), q, po, pml); break;
    case 2: hipLaunchKernelGGL(asv::attn_split<2>, grid, block, 0, st, tv, int(layer), q, po, pml); break;
    case 3: hipLaunchKernelGGL(asv::attn_split<3>, grid, block, 0, st, tv, int(layer), q, po, pml); break;
    default: hipLaunchKernelGGL(asv::attn_split<4>, grid, block, 0, st, tv, int(layer), q, po, pml); break;
  }
  return hipGetLastError() == hipSuccess ? ASV_OK : ASV_E_HIP;
}

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
  hipLaunchKernelGGL(asv::merge_rows, dim3((pairs + 15) / 16), dim3(256), 0,
                     static_cast<hipStream_t>(stream), tv, po, pml, o);
  return hipGetLastError() == hipSuccess ? ASV_OK : ASV_E_HIP;
}
