// Split-K GQA attention over every stream of a shared round, and the merge
// of each row's split partials (gfx950).
//
// PR #1377 "LFM2: shared-round decode", shared-round commit: one attention
// launch a layer covers every stream's rows through the segment table; each
// stream's partials are held apart in the scratch; one merge launch follows.
// The per-record arithmetic is written out in include/asv.h.
//
// Work item = (16-row tile, kv head, split), one 256-thread block each. A
// tile's q vectors are its rows x the 4 q heads of the kv head (up to 64),
// in column tiles of 16. The block's 4 waves load each 128-key stage of K
// and V together into an LDS ring (two stages in flight in registers) and
// then split the work: 16-row tiles give each wave one q tile over every
// key; smaller tiles split the keys between waves, which fold their states
// through LDS in a fixed order at the end.
//
// Per 32-key sub-block, on the bf16 16x16x32 MFMA (fp32 accumulate):
//   S^T[key][q]  = K[key][:] . Q[q][:]        (2 key tiles x 2 d-steps)
//   O^T[d][q]   += V^T[d][key] P^T[key][q]    (4 d tiles, P split hi + lo)
// K rows are key-major in HBM, V is d-major inside 32-key blocks, and the
// LDS ring holds both in MFMA operand order, so each operand is one
// conflict-free 16-byte LDS read.
//
// Lane l (G = l/16, c = l%16) of a score tile holds keys 8G+i (first tile)
// and 8G+4+i (second tile), i = 0..3, for q column c: the stage's K rows are
// placed so that these 8 keys are exactly the ones the lane supplies as the
// P operand of the PV MFMA, whose V operand is V^T[d][8G..8G+7]. P is fed
// as two bf16 parts (hi = the top 16 bits of the fp32 weight, lo = the
// rest) so the partials keep ~16 bits of the weights, not bf16's 8.
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

__device__ __forceinline__ uint32_t zero_past(uint32_t w, int key, int keys) {
  if (key >= keys) w &= 0xFFFF0000u;
  if (key + 1 >= keys) w &= 0x0000FFFFu;
  return w;
}

// Per-wave online-softmax state for QPW q tiles. The wave keeps, per q
// column, a reference max mref (the exponent base) and the true running max
// mtrue. mref moves only when a block's max exceeds it by more than kLazy in
// log2 units, so the accumulators are rescaled rarely (weights stay below
// 2^kLazy); at the end l is brought to the true max, which a record holds.
template <int QPW>
struct WaveState {
  f32x4 acc[4][QPW];
  float mref[QPW], mtrue[QPW], l[QPW];
};

constexpr float kLazy = 8.0f;

// A stage is 128 keys of one kv head: four 32-key sub-blocks, each K 4 KB +
// V 4 KB. The block's 256 threads load a stage together (thread t: 16 bytes
// of K and 16 of V of every sub-block, each wave reading 1 KB contiguous)
// two stages ahead, and store it into an LDS slot in MFMA operand order:
// inside a sub-block, K operand (tile X, d-step s) of lane l sits at
// ((2X + s)*64 + l)*16 bytes and V operand (d tile dt) of lane l at
// 4096 + (dt*64 + l)*16, so each operand read is a conflict-free
// ds_read_b128 at lane*16.
constexpr int kStageKeys = 128;
constexpr int kSubBytes = 8192;
constexpr int kStageBytes = 4 * kSubBytes;

#ifndef ASV_ATTN_REG_STAGES
#define ASV_ATTN_REG_STAGES 2
#endif
constexpr int kRegStages = ASV_ATTN_REG_STAGES;  // stages in flight in registers

struct StageRegs {
  u32x4 k[4], v[4];
};

__device__ __forceinline__ void stage_load(StageRegs& r, const uint16_t* __restrict__ Kh,
                                           const uint16_t* __restrict__ Vh, int ks, int last_sb,
                                           int t) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // sub-blocks past the split's last one re-read that one (a cache hit):
    // every stage issues the same loads, so waits stay exact
    const int sb = min(ks + 32 * j, last_sb);
    r.k[j] = load16_stream(Kh + int64_t(sb + (t >> 3)) * ASV_HEAD_DIM + (t & 7) * 8);
    r.v[j] = load16_stream(Vh + int64_t(sb >> 5) * (ASV_HEAD_DIM * 32) + t * 8);
  }
}

// Operand slot of lane l inside a 64-lane group, XOR-swizzled within its
// 16-lane block (lane c of block G goes to c ^ 2G ^ x). Readers stay a
// permutation of 256 contiguous bytes per 16 lanes (conflict-free); a
// store pass (one K row's 8 chunks, or 2 d-rows x 4 key groups of V) now
// spreads over all 8 16-byte slots of a 128-byte bank row.
__device__ __forceinline__ int swz(int l, int x) { return (l & 48) | ((l & 15) ^ ((l >> 3) & 6) ^ x); }

__device__ __forceinline__ void stage_store(const StageRegs& r, char* slot, int kofs, int vofs) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    *reinterpret_cast<u32x4*>(slot + j * kSubBytes + kofs) = r.k[j];
    *reinterpret_cast<u32x4*>(slot + j * kSubBytes + vofs) = r.v[j];
  }
}

// One 32-key sub-block for QPW q tiles; operands come from LDS.
template <int QPW>
__device__ __forceinline__ void sub_block(const char* sub, int kb, int keys, int n_first,
                                          const u32x4 (&qop)[QPW][2], const int (&nq)[QPW],
                                          WaveState<QPW>& st, int lane) {
  const int G = lane >> 4;
  const float c = kScale * kLog2e;
  const float lazy_raw = kLazy / c;
  const float ninf = -__builtin_inff();
  const int l0 = swz(lane, 0), l1 = swz(lane, 1);
  const u32x4 ka0 = *reinterpret_cast<const u32x4*>(sub + (0 * 64 + l0) * 16);
  const u32x4 ka1 = *reinterpret_cast<const u32x4*>(sub + (1 * 64 + l1) * 16);
  const u32x4 kb0 = *reinterpret_cast<const u32x4*>(sub + (2 * 64 + l0) * 16);
  const u32x4 kb1 = *reinterpret_cast<const u32x4*>(sub + (3 * 64 + l1) * 16);
  u32x4 v[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) v[dt] = *reinterpret_cast<const u32x4*>(sub + 4096 + (dt * 64 + l0) * 16);
  if (kb + 32 > keys) {  // slots past the key count may hold anything
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int w = 0; w < 4; ++w) v[dt][w] = zero_past(v[dt][w], kb + 8 * G + 2 * w, keys);
  }
  const bool edge = kb + 32 > n_first;
#pragma unroll
  for (int u = 0; u < QPW; ++u) {
    f32x4 sa = mfma(ka0, qop[u][0], f32x4{0.f, 0.f, 0.f, 0.f});
    sa = mfma(ka1, qop[u][1], sa);
    f32x4 sb = mfma(kb0, qop[u][0], f32x4{0.f, 0.f, 0.f, 0.f});
    sb = mfma(kb1, qop[u][1], sb);
    float sc[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
    if (edge) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (kb + 8 * G + jj >= nq[u]) sc[jj] = ninf;
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                     fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mx = max_xor32(max_xor16(mx));
    st.mtrue[u] = fmaxf(st.mtrue[u], mx);
    const bool move = mx > st.mref[u] + lazy_raw;
    if (__any(move)) {  // wave-uniform; x * 1.0f leaves the other columns' bits unchanged
      const float alpha = move ? exp2_((st.mref[u] - mx) * c) : 1.f;
      st.mref[u] = move ? mx : st.mref[u];
      st.l[u] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) st.acc[dt][u] *= alpha;
    }
    const float nmc = -((st.mref[u] == ninf) ? 0.f : st.mref[u]) * c;
    float p[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) p[jj] = exp2_(__builtin_fmaf(sc[jj], c, nmc));
    st.l[u] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    u32x4 hi, lo;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // hi = top halves of two weights in one v_perm_b32; lo = what they drop
      const uint32_t a = __float_as_uint(p[2 * w]);
      const uint32_t b = __float_as_uint(p[2 * w + 1]);
      hi[w] = __builtin_amdgcn_perm(b, a, 0x07060302u);
      const float ra = p[2 * w] - __uint_as_float(a & 0xFFFF0000u);
      const float rb = p[2 * w + 1] - __uint_as_float(b & 0xFFFF0000u);
      lo[w] = __builtin_amdgcn_perm(__float_as_uint(rb), __float_as_uint(ra), 0x07060302u);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      st.acc[dt][u] = mfma(v[dt], hi, st.acc[dt][u]);
      st.acc[dt][u] = mfma(v[dt], lo, st.acc[dt][u]);
    }
  }
}

// Fold state b into a (a first, then b: the order is fixed).
template <int QPW>
__device__ __forceinline__ void fold(WaveState<QPW>& a, float mref_b, float mtrue_b, float l_b,
                                     const f32x4* acc_b, int u) {
  const float c = kScale * kLog2e;
  const float ninf = -__builtin_inff();
  const float mn = fmaxf(a.mref[u], mref_b);
  const float base = (mn == ninf) ? 0.f : mn;
  const float a0 = exp2_((a.mref[u] - base) * c);
  const float a1 = exp2_((mref_b - base) * c);
  a.mref[u] = mn;
  a.mtrue[u] = fmaxf(a.mtrue[u], mtrue_b);
  a.l[u] = __builtin_fmaf(l_b, a1, a.l[u] * a0);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_fmaf(acc_b[dt][i], a1, a.acc[dt][u][i] * a0);
    a.acc[dt][u] = r;
  }
}

// A block of 4 waves runs one work item. The waves load every stage
// together; for computing they split the item's q tiles into QG groups of
// QPW tiles and each stage's four sub-blocks into KG = 4/QG interleaved
// groups (wave (qg, kg) takes sub-blocks kg, kg+KG, ...). A q group's waves
// fold their states through LDS in key-group order at the end.
template <int QPW>
__device__ __forceinline__ void attn_item(const TableView& tv, int layer,
                                          const uint16_t* __restrict__ Q, float* __restrict__ po,
                                          float* __restrict__ pml, const asv_work wk, int nqt,
                                          char* __restrict__ lds) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int G = lane >> 4;
  const int c16 = lane & 15;
  const asv_tile T = uniform(cload(tv.tiles + wk.tile));
  const asv_seg S = uniform(cload(tv.segs + T.stream));
  const int g = wk.head;
  // q groups: 1 (one q tile), 2 (two), 4 (three or four; a fourth group
  // with no rows only helps load)
  const int QG = (nqt >= 3) ? 4 : nqt;
  const int KG = kWaves / QG;
  const int qg = wave / KG;
  const int kg = wave - qg * KG;
  const int base_n = S.keys - S.rows + T.pos0;  // tile row i sees base_n + i + 1 keys
  const int n_first = base_n + 1;
  const int k0 = wk.split * S.split_keys;
  const int k1 = min(k0 + S.split_keys, base_n + T.nrows);
  const int last_sb = ((k1 - 1) >> 5) << 5;
  const int64_t head_elems = int64_t(S.cap) * ASV_HEAD_DIM;
  const int64_t sel = int64_t(layer) * tv.n_streams + T.stream;
  const uint16_t* Kh = reinterpret_cast<const uint16_t*>(uniform_ptr(cload(tv.kp + sel))) + g * head_elems;
  const uint16_t* Vh = reinterpret_cast<const uint16_t*>(uniform_ptr(cload(tv.vp + sel))) + g * head_elems;

  // Q operands (B of the score MFMA) and each column's visible key count
  WaveState<QPW> st;
  u32x4 qop[QPW][2];
  int nq[QPW];
  const float ninf = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < QPW; ++u) {
    const int q = (qg * QPW + u) * 16 + c16;
    const int rt = q >> 2;
    if (rt < T.nrows) {
      const uint16_t* qp =
          Q + (int64_t(T.row0 + rt) * ASV_Q_HEADS + g * 4 + (q & 3)) * ASV_HEAD_DIM + 8 * G;
      qop[u][0] = load16(qp);
      qop[u][1] = load16(qp + 32);
      nq[u] = base_n + rt + 1;
    } else {
      qop[u][0] = u32x4{0u, 0u, 0u, 0u};
      qop[u][1] = u32x4{0u, 0u, 0u, 0u};
      nq[u] = 0;
    }
    st.mref[u] = ninf;
    st.mtrue[u] = ninf;
    st.l[u] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.acc[dt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const bool active = qg * QPW * 16 < T.nrows * 4;  // the group holds a real q column

  // where this thread's 16-byte pieces of a sub-block go in operand order
  int kofs, vofs;
  {
    const int kk = t >> 3, ch = t & 7;  // K: key kk, 16-byte chunk ch of its row
    const int X = (kk >> 2) & 1, m = ((kk >> 3) << 2) | (kk & 3), sd = ch >> 2;
    kofs = ((2 * X + sd) * 64 + swz((ch & 3) * 16 + m, sd)) * 16;
    const int d = t >> 2;               // V: dim d, keys 8*(t&3) .. +7
    vofs = 4096 + ((d >> 4) * 64 + swz((t & 3) * 16 + (d & 15), 0)) * 16;
  }

  // stages in flight: kRegStages in registers while one is consumed from
  // LDS; two LDS slots, one barrier a stage (a slot is rewritten only after
  // every wave has passed the barrier that follows its last read)
  const int nst = (k1 - k0 + kStageKeys - 1) / kStageKeys;
  StageRegs r[kRegStages];
#pragma unroll
  for (int h = 0; h < kRegStages; ++h)
    stage_load(r[h], Kh, Vh, k0 + min(h, nst - 1) * kStageKeys, last_sb, t);
  // Every step of an iteration stores, prefetches (clamped) and passes the
  // barrier, so every iteration leaves the same loads in flight and the wait
  // before a store covers only that stage; steps past the last stage skip
  // their compute.
  for (int i = 0; i < nst; i += kRegStages) {
#pragma unroll
    for (int h = 0; h < kRegStages; ++h) {
      const int si = i + h;
      char* slot = lds + (si & 1) * kStageBytes;
      stage_store(r[h], slot, kofs, vofs);
      stage_load(r[h], Kh, Vh, k0 + min(si + kRegStages, nst - 1) * kStageKeys, last_sb, t);
      __syncthreads();
      const int ks = k0 + si * kStageKeys;
      if (!active || si >= nst) continue;
      for (int sbi = kg; sbi < 4; sbi += KG) {
        const int kb = ks + 32 * sbi;
        if (kb >= k1) break;
        sub_block<QPW>(slot + sbi * kSubBytes, kb, S.keys, n_first, qop, nq, st, lane);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < QPW; ++u) st.l[u] = add_xor32(add_xor16(st.l[u]));
  __syncthreads();  // the ring is reused for the fold

  // fold the key groups of each q group in order through LDS
  float* fl = reinterpret_cast<float*>(lds);
  constexpr int kSlot = QPW * 64 * 19;  // mref, mtrue, l, then 4 x QPW f32x4 per lane
  if (kg > 0) {
    float* my = fl + (qg * (kWaves - 1) + kg - 1) * kSlot;
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
      my[u * 64 + lane] = st.mref[u];
      my[(QPW + u) * 64 + lane] = st.mtrue[u];
      my[(2 * QPW + u) * 64 + lane] = st.l[u];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        *reinterpret_cast<f32x4*>(my + 3 * QPW * 64 + ((dt * QPW + u) * 64 + lane) * 4) = st.acc[dt][u];
    }
  }
  __syncthreads();
  if (kg != 0) return;
  for (int w = 1; w < KG; ++w) {
    const float* o = fl + (qg * (kWaves - 1) + w - 1) * kSlot;
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
      f32x4 accb[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        accb[dt] = *reinterpret_cast<const f32x4*>(o + 3 * QPW * 64 + ((dt * QPW + u) * 64 + lane) * 4);
      fold<QPW>(st, o[u * 64 + lane], o[(QPW + u) * 64 + lane], o[(2 * QPW + u) * 64 + lane], accb, u);
    }
  }

  // records: o = acc / l (any exponent base), then (true max in score units,
  // l taken to the true max)
  const float c = kScale * kLog2e;
#pragma unroll
  for (int u = 0; u < QPW; ++u) {
    const int q = (qg * QPW + u) * 16 + c16;
    const int rt = q >> 2;
    if (rt >= T.nrows) continue;
    const int64_t rec =
        S.poff + (int64_t(wk.split) * S.rows + T.pos0 + rt) * ASV_Q_HEADS + g * 4 + (q & 3);
    const float L = st.l[u];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (L > 0.f) ? st.acc[dt][u][i] / L : 0.f;
      store16f(po + rec * ASV_HEAD_DIM + dt * 16 + 4 * G, r);
    }
    if (G == 0) {
      const float mt = st.mtrue[u];
      const float lt = (mt == ninf) ? 0.f : L * exp2_((st.mref[u] - mt) * c);
      gstore(reinterpret_cast<float2*>(pml) + rec, make_float2((mt == ninf) ? ninf : mt * kScale, lt));
    }
  }
}

template <int QPW_MAX>
__global__ __launch_bounds__(kThreads, 2) void attn_split(TableView tv, int layer,
                                                          const uint16_t* __restrict__ Q,
                                                          float* __restrict__ po,
                                                          float* __restrict__ pml) {
  // two stage slots (64 KB); the fold area after the loop reuses them
  __shared__ __attribute__((aligned(16))) char lds[2 * kStageBytes];
  const asv_work wk = uniform(cload(tv.work + blockIdx.x));
  const int nqt = (uni(cload(tv.tiles + wk.tile).nrows) + 3) >> 2;
  attn_item<QPW_MAX>(tv, layer, Q, po, pml, wk, nqt, lds);
}

// Merge: one wave per (row, q head); lane d owns output dim d. The wave
// first takes M = max_t m_t over the row's splits (lanes over splits), then
// every lane walks the splits in order, t = 0, 1, ..., adding
// w_t = e^(m_t - M) l_t and w_t o_t[d]; the loads of successive splits are
// independent, so they stay in flight together.
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
  const int nt = (row.nkeys + S.split_keys - 1) / S.split_keys;
  const int64_t rec0 = S.poff + int64_t(row.pos) * ASV_Q_HEADS + h;
  const int64_t step = int64_t(S.rows) * ASV_Q_HEADS;
  const float2* ml = reinterpret_cast<const float2*>(pml);
  const float ninf = -__builtin_inff();

  float M = ninf;
  for (int t = lane; t < nt; t += 64) {
    const float2 v = gload(ml + rec0 + t * step);
    if (v.y != 0.f) M = fmaxf(M, v.x);  // empty splits (l = 0) take no part
  }
  M = wave_max(M);

  float L = 0.f, acc = 0.f;
  const float* o = po + rec0 * ASV_HEAD_DIM + lane;
  const int64_t ostep = step * ASV_HEAD_DIM;
#pragma unroll 4
  for (int t = 0; t < nt; ++t) {
    const float2 v = gload(ml + rec0 + t * step);
    const float ot = gload(o + t * ostep);
    if (v.y == 0.f) continue;  // empty split; a NaN partial falls through and propagates
    const float w = exp2_((v.x - M) * kLog2e) * v.y;
    L += w;
    acc = __builtin_fmaf(w, ot, acc);
  }
  const float y = (L != 0.f) ? acc / L : 0.f;
  gstore(O + (int64_t(r) * ASV_Q_HEADS + h) * ASV_HEAD_DIM + lane, uint16_t(f32_to_bf16(y)));
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
  hipLaunchKernelGGL(asv::attn_split<1>, grid, block, 0, st, tv, int(layer), q, po, pml);
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
  hipLaunchKernelGGL(asv::merge_rows, dim3((pairs + asv::kMergeWaves - 1) / asv::kMergeWaves),
                     dim3(64 * asv::kMergeWaves), 0,
                     static_cast<hipStream_t>(stream), tv, po, pml, o);
  return hipGetLastError() == hipSuccess ? ASV_OK : ASV_E_HIP;
}
