// Split-K GQA attention over every stream of a shared round (gfx950); the
// merge of each row's split partials is in merge.hip.
//
// PR #1377 "LFM2: shared-round decode", shared-round commit: one attention
// launch a layer covers every stream's rows through the segment table; each
// stream's partials are held apart in the scratch; one merge launch follows
// (merge.hip).
// The per-record arithmetic is written out in include/asv.h.
//
// Work item = (16-row tile, kv head, split), one 256-thread block each. A
// tile's q vectors are its rows x the 4 q heads of the kv head (up to 64),
// in column tiles of 16. Every wave of the block holds all of the tile's q
// tiles (their Q operands in registers) and streams its own quarter of the
// split's keys (32-key sub-blocks w, w+4, ...) through a private LDS ring
// that direct global->LDS loads fill; at the end the four waves fold their
// states through LDS in wave order. Streams of more than one tile (prompt
// chunks) are split into group items instead: up to four consecutive tiles,
// one a wave, that walk the split's keys together through one shared ring
// (attn_group below).
//
// Per 32-key sub-block, on the 16x16x32 MFMA (fp32 accumulate):
//   S^T[key][q]  = K[key][:] . Q[q][:]        (bf16; 2 key tiles x 2 d-steps)
//   O^T[d][q]   += V^T[d][key] P^T[key][q]    (4 d tiles: bf16 with P split
//                                              hi + lo, or fp16 for groups)
// K rows are key-major in HBM, V is d-major inside 32-key blocks; each
// operand is one conflict-free 16-byte LDS read.
//
// Lane l (G = l/16, c = l%16) of a score tile holds keys 8G+i (first tile)
// and 8G+4+i (second tile), i = 0..3, for q column c: the K rows are
// placed so that these 8 keys are exactly the ones the lane supplies as the
// P operand of the PV MFMA, whose V operand is V^T[d][8G..8G+7]. P is fed
// as two bf16 parts (hi = the top 16 bits of the fp32 weight, lo = the
// rest) so the partials keep ~16 bits of the weights, not bf16's 8.
//
// Group items run the PV product on the fp16 MFMA instead, one MFMA a d
// tile: each wave rewrites its quarter of every V sub-block in LDS as fp16
// under a power-of-2 scale of its d tile that follows the values' size
// (exact for every finite bf16 value down to 2^-22 of its sub-block's
// largest; convert_quarter), and the weights are rounded to fp16 (11 bits:
// relative error at most 2^-11 each, the same rounded weights in l and in
// o). This halves the MFMAs of the product, where the chunks' arithmetic
// goes, at a cost in the partials' error: about 5e-4 of a record's largest
// |o| at most on the test workloads, where bf16 hi + lo stays near 2e-5.
//
// Bits depend only on the item's own stream: the split plan and the grouping
// of its tiles come from the stream's rows and keys, each item writes its
// own records, and the fold order is fixed, so a shared round gives the same
// bits as each stream run alone.

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

// The fp16 form of the same product, for group items whose V sub-block fits
// fp16 exactly (see convert_quarter).
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t zero_past(uint32_t w, int key, int keys) {
  if (key >= keys) w &= 0xFFFF0000u;
  if (key + 1 >= keys) w &= 0x0000FFFFu;
  return w;
}

// Per-wave online-softmax state for QPW q tiles. Per q column the wave
// keeps an exponent base mref (raw score units; -inf until the column has
// seen a key), nmc = -mref*c, the sum l of its weights at that base (summed
// by the MFMA, see accumulate: all four entries hold the column's sum), the
// largest score ms it has seen, and thr = mref + kLazy/c. A sub-block's
// scores are tested against thr first; only when one of them exceeds it (a
// weight above 2^kLazy at the current base), or on the wave's first
// sub-block, does the wave take the rebase path, which moves the bases to
// the columns' max scores and rescales. So the common path has no cross-lane
// max at all, and the accumulators are rescaled rarely. At the end the true
// max is the largest score seen, and l is taken to it.
template <int QPW>
struct WaveState {
  f32x4 acc[4][QPW];
  f32x4 l[QPW];
  float mref[QPW], nmc[QPW], thr[QPW], ms[QPW];
  uint32_t ev;  // group items: byte dt = the V scale exponent of d tile dt + 112
};

// Loop-invariant operands of accumulate, each held in registers: a ones
// matrix (bf16 1.0 in every element) and the bf16 pairs (-1, 0), (0, -1).
// They pass through an empty asm so the compiler cannot turn them into
// inline constants: as the packed-bf16 operand of v_dot2c_f32_bf16 it
// would encode (-1, 0) as the 32-bit constant -1.0, which the hardware
// reads as the pair (0, -1).
struct Consts {
  u32x4 ones;
  uint32_t neg_lo, neg_hi;
};

__device__ __forceinline__ Consts make_consts() {
  Consts k;
  uint32_t one = 0x3F803F80u, a = 0x0000BF80u, b = 0xBF800000u;
  asm volatile("" : "+v"(one), "+v"(a), "+v"(b));
  k.ones = u32x4{one, one, one, one};
  k.neg_lo = a;
  k.neg_hi = b;
  return k;
}

constexpr float kLazy = 8.f;  // weights stay <= 2^8 between rebases
// Group items round the weights to fp16 taken 2^7 times their value (at
// most 2^15 then): fp16's normal range then holds every weight down to
// 2^-21 of the base with its full 11 bits, below which a weight keeps bits
// down to 2^-31 of the base only.
constexpr int kPShift16 = 7;

// Each wave streams its own 32-key sub-blocks (the item's sub-blocks w,
// w+4, w+8, ... for wave w) through a private two-slot LDS ring filled by
// direct global->LDS loads (global_load_lds_dwordx4): no registers hold data
// in flight and no block barrier paces the waves. A load instruction puts
// lane l's 16 bytes at (its 1 KB group) + l*16, and every instruction reads
// one whole 1 KB run of HBM (lanes may take its 16-byte chunks in any order
// at full speed; instructions that cover half-lines of 16 rows run ~15%
// slower). Group j of K holds key rows 8j..8j+7 with the chunks permuted so
// that the score MFMA's operand reads hit 16 distinct 16-byte bank groups
// per 16 lanes (k_fetch / k_read below); group 4+dt of V holds V^T rows
// 16dt..16dt+15, which is already one 1 KB run in the d-major V layout:
// lane (G, c) fetches the operand it reads back, V^T[16dt + c][8G..8G+7].
// 8 KB a slot.
constexpr int kSubBytes = 8192;

// Score-MFMA lane (G, c) supplies, for key tile X and d-step s, key row
// 8(c>>2) + 4X + (c&3), d-columns 8(4s+G)..+7: row 4X + (c&3) of K group
// j = c>>2. k_fetch gives the byte offset, inside group j (key rows
// 8j..8j+7, 128 B each), of the 16-byte chunk lane l fetches; bits of l:
// b5 = X, b4 = G>>1, b3 = (G&1)^(j>>1), b2 = s^(j&1), b1b0 = (c&3)^G.
__device__ __forceinline__ uint32_t k_fetch(int l, int j) {
  const int G = (((l >> 4) & 1) << 1) | (((l >> 3) & 1) ^ ((j >> 1) & 1));
  const int s = ((l >> 2) & 1) ^ (j & 1);
  const int r = 4 * ((l >> 5) & 1) + ((l & 3) ^ G);
  return uint32_t(r * 128 + (4 * s + G) * 16);
}

// LDS byte offset (within a slot) of the K operand of score-MFMA lane
// (G, c) for key tile X = 0 and d-step s; key tile 1 is 512 bytes on.
__device__ __forceinline__ uint32_t k_read(int G, int c, int s) {
  const int j = c >> 2;
  const int l = ((G >> 1) << 4) | (((G & 1) ^ (j >> 1)) << 3) | ((s ^ (j & 1)) << 2) | ((c & 3) ^ G);
  return uint32_t(j * 1024 + l * 16);
}

// 16 bytes from (wave-uniform base + per-lane byte offset) to LDS at
// l + lane*16. The offset is passed through an opaque register copy so the
// compiler keeps it a 32-bit register next to a scalar base (the
// scalar-base form of global_load_lds_dwordx4) instead of hoisting a 64-bit
// per-lane address for every load out of the loop.
// AUX is the load's cache policy: kStream (non-temporal) for K/V that one
// work item alone reads, 0 where several tiles of a stream re-read it. IMM
// is the instruction's immediate offset, which moves the global and the LDS
// address alike.
template <int AUX, int IMM = 0>
__device__ __forceinline__ void lds_dma16(const char* base, uint32_t off, void* l) {
  uint32_t o;
  asm volatile("v_mov_b32 %0, %1" : "=v"(o) : "v"(off));
  const ASV_GLOBAL char* b = (const ASV_GLOBAL char*)(base);
  __builtin_amdgcn_global_load_lds((const ASV_GLOBAL void*)(b + o),
                                   (__attribute__((address_space(3))) void*)(l), 16, IMM, AUX);
}

constexpr int kStream = 2;  // the nt bit of the cache-policy operand

// Wait until at most n vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int AUX>
__device__ __forceinline__ void issue_sub(char* slot, const uint16_t* __restrict__ Kh,
                                          const uint16_t* __restrict__ Vh, int kb,
                                          const uint32_t (&koff)[4], uint32_t voff) {
  const char* kbase = reinterpret_cast<const char*>(Kh + int64_t(kb) * ASV_HEAD_DIM);
  const char* vbase = reinterpret_cast<const char*>(Vh + int64_t(kb >> 5) * (ASV_HEAD_DIM * 32));
#pragma unroll
  for (int j = 0; j < 4; ++j) lds_dma16<AUX>(kbase, koff[j], slot + j * 1024);
  lds_dma16<AUX, 0>(vbase, voff, slot + 4096);
  lds_dma16<AUX, 1024>(vbase, voff, slot + 4096);
  lds_dma16<AUX, 2048>(vbase, voff, slot + 4096);
  lds_dma16<AUX, 3072>(vbase, voff, slot + 4096);
}

// Max of three scores on gfx950's v_maximum3_f32 (a NaN propagates). fmaxf
// would first quiet every MFMA result with an extra v_max_f32 x, x.
__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Rebase q tile u (wave-uniform, rare): every column moves its base up to
// its max score so far (ms: the lane's max of every score it has seen);
// x * 1.0f leaves the bits of columns that do not move unchanged. PSHIFT: weights
// are taken 2^PSHIFT times their value at the base (l and o alike, so o is
// unchanged and l is divided back at the end).
template <int QPW, int PSHIFT = 0>
__device__ __forceinline__ void rebase(WaveState<QPW>& st, int u, float ms) {
  const float c = kScale * kLog2e;
  const float ninf = -__builtin_inff();
  const float mx = max_xor32(max_xor16(ms));
  const float mn = fmaxf(st.mref[u], mx);
  const float alpha = (mn > st.mref[u]) ? exp2_((st.mref[u] - mn) * c) : 1.f;
  st.mref[u] = mn;
  st.nmc[u] = (mn == ninf) ? 0.f : -mn * c + float(PSHIFT);
  st.thr[u] = mn + kLazy / c;
  st.l[u] *= alpha;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) st.acc[dt][u] *= alpha;
}

// q tile u's scores (in place: their weights at the current base), as bf16
// hi + lo, through the PV MFMAs into the accumulators, and through two more
// MFMAs with a ones matrix into l: the sum over the sub-block's 32 keys of
// every column lands in all four entries, so l costs no VALU adds and no
// reduction across lanes at the end.
template <int QPW>
__device__ __forceinline__ void accumulate(WaveState<QPW>& st, int u, float (&p)[8],
                                           const u32x4 (&v)[4], const Consts& kc) {
  const float c = kScale * kLog2e;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) p[jj] = exp2_(__builtin_fmaf(p[jj], c, st.nmc[u]));
  u32x4 hi, lo;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    // hi = top halves of two weights in one v_perm_b32; what they drop is
    // p - hi, exact in fp32, one v_dot2c_f32_bf16 each (hi . (-1, 0) + p)
    // (the pair is bit-cast from a plain local: a bit cast of the vector
    // element hi[w] inside this unrolled loop was compiled as hi[0] for
    // every w)
    const uint32_t h =
        __builtin_amdgcn_perm(__float_as_uint(p[2 * w + 1]), __float_as_uint(p[2 * w]), 0x07060302u);
    hi[w] = h;
    const bf16x2 hb = __builtin_bit_cast(bf16x2, h);
    const float ra =
        __builtin_amdgcn_fdot2_f32_bf16(hb, __builtin_bit_cast(bf16x2, kc.neg_lo), p[2 * w], false);
    const float rb = __builtin_amdgcn_fdot2_f32_bf16(hb, __builtin_bit_cast(bf16x2, kc.neg_hi),
                                                     p[2 * w + 1], false);
    lo[w] = __builtin_amdgcn_perm(__float_as_uint(rb), __float_as_uint(ra), 0x07060302u);
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    st.acc[dt][u] = mfma(v[dt], hi, st.acc[dt][u]);
    st.acc[dt][u] = mfma(v[dt], lo, st.acc[dt][u]);
  }
  st.l[u] = mfma(kc.ones, hi, st.l[u]);
  st.l[u] = mfma(kc.ones, lo, st.l[u]);
}

// accumulate for a sub-block whose V operands hold fp16: the weights are
// rounded to fp16 (one v_cvt_pk_f16_f32 a pair, relative error <= 2^-11),
// and the same rounded weights go through one PV MFMA per d tile and one l
// MFMA, so o = acc / l stays an exact weighted mean of V under the rounded
// weights.
template <int QPW>
__device__ __forceinline__ void accumulate16(WaveState<QPW>& st, int u, float (&p)[8],
                                             const u32x4 (&v)[4], const u32x4& ones16) {
  const float c = kScale * kLog2e;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) p[jj] = exp2_(__builtin_fmaf(p[jj], c, st.nmc[u]));
  u32x4 ph;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x2 f = {p[2 * w], p[2 * w + 1]};
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
    ph[w] = h;
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) st.acc[dt][u] = mfma16(v[dt], ph, st.acc[dt][u]);
  st.l[u] = mfma16(ones16, ph, st.l[u]);
}

// Scores of q tile u over the sub-block's 32 keys: lane (G, c) gets, for q
// column c, keys 8G .. 8G+7 (the first four from key tile 0, the last four
// from key tile 1). EDGE: keys at or past the column's visible count are
// set to -inf.
template <int QPW, bool EDGE>
__device__ __forceinline__ void scores(const u32x4 (&k)[4], const u32x4 (&qop)[QPW][2], int u,
                                       int kb, int G, const int (&nq)[QPW], float (&sc)[8]) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 sa = mfma(k[0], qop[u][0], z);
  f32x4 sb = mfma(k[2], qop[u][0], z);
  sa = mfma(k[1], qop[u][1], sa);
  sb = mfma(k[3], qop[u][1], sb);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = sa[i];
    sc[4 + i] = sb[i];
  }
  if constexpr (EDGE) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      if (kb + 8 * G + jj >= nq[u]) sc[jj] = -__builtin_inff();
  }
}

// LDS reads the compiler does not see, for the shared ring of group items:
// its slot is chosen at run time, so the compiler cannot tell the slot being
// read from the ones the direct loads are filling, and before a plain read
// it would wait for every load in flight (vmcnt(0)). Each statement waits
// for its own reads' results (lgkmcnt(0)) before it ends.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return uint32_t(size_t((__attribute__((address_space(3))) const char*)(p)));
}

// K operands: rows at a0 and a1 (d-steps 0 and 1), key tile 1 512 bytes on;
// with them the 16 bytes at aq (this lane's part of the next sub-block's
// quarter, which the wave converts) and the word at aw (the slot's exponent
// word), all under one wait.
__device__ __forceinline__ void lds_read_k_q(u32x4 (&k)[4], u32x4& q, uint32_t& w, uint32_t a0,
                                             uint32_t a1, uint32_t aq, uint32_t aw) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b128 %2, %6 offset:512\n\t"
      "ds_read_b128 %3, %7 offset:512\n\t"
      "ds_read_b128 %4, %8\n\t"
      "ds_read_b32 %5, %9\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(q), "=&v"(w)
      : "v"(a0), "v"(a1), "v"(aq), "v"(aw)
      : "memory");
}

// V operands of the four d tiles, 1 KB apart from a
__device__ __forceinline__ void lds_read_v(u32x4 (&v)[4], uint32_t a) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\t"
      "ds_read_b128 %3, %4 offset:3072\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a)
      : "memory");
}

// Largest u32 over the wave: DPP within rows of 16 lanes, then across rows.
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  auto dmax = [](uint32_t v, uint32_t o) { return v > o ? v : o; };
  x = dmax(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0xB1, 0xF, 0xF, false)));   // lane ^ 1
  x = dmax(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x4E, 0xF, 0xF, false)));   // lane ^ 2
  x = dmax(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x141, 0xF, 0xF, false)));  // 7 - i in 8
  x = dmax(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x140, 0xF, 0xF, false)));  // 15 - i
  x = umax_xor16(x);
  x = umax_xor32(x);
  return uint32_t(__builtin_amdgcn_readfirstlane(int(x)));
}

// A wave's V exponent for its d tile, and the lowest it has taken in the item.
struct VScale {
  int e = 142, emin = 142;
};

// Wave w's pass over its own quarter of a landed sub-block (d tile w of V,
// all 32 keys: the 16 bytes each lane loaded itself), before the block
// barrier. V past the key count is zeroed; the quarter is then scaled by 2^e
// and rewritten in place as fp16. e is the wave's exponent for its d tile,
// which follows the quarters' largest finite magnitudes: with E the bf16
// exponent field of a quarter's largest, 142 - E puts it below 2^16. e is
// lowered to that when the quarter does not fit, and raised to it (at most
// 64 above the lowest e of the item, so the accumulators cannot overflow
// when they follow) when every magnitude of the quarter is below 2^-8 of
// what e allows; otherwise it stays. Every finite value so lands on an fp16
// number exactly (8 significant bits) unless it falls below 2^-14 after
// scaling, which is 2^-22 of its quarter's largest or less (unless the cap
// held e down).
// When the quarter fits the current e (the common case) the conversion is
// integer arithmetic on the bf16 bits: magnitude minus (112 - e) << 7,
// saturating at zero, shifted left by 3, with the sign put back; values
// below 2^-14 after scaling then come out zero or off by less than 2^-14.
// Otherwise (e moves, or Inf or NaN present, or e > 112) it goes through
// fp32 (v_ldexp_f32, then v_cvt_pk_f16_f32), which keeps bits down to
// 2^-24 after scaling, and Inf and NaN stay Inf and NaN. e + 112 goes to
// byte w of the slot's exponent word.
//
// convert_quarter takes the 16 bytes already read from LDS address a, where
// it writes them back.
__device__ __forceinline__ void convert_quarter(u32x4 x, uint32_t a, uint32_t word_addr, int wave,
                                                int lane, int kb, int keys, VScale& vs) {
  if (kb + 32 > keys) {
#pragma unroll
    for (int w = 0; w < 4; ++w) x[w] = zero_past(x[w], kb + 8 * (lane >> 4) + 2 * w, keys);
  }
  u16x2 mx = {0, 0};
  u16x2 mag[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t m = x[w] & 0x7FFF7FFFu;
    mag[w] = __builtin_bit_cast(u16x2, m);
    mx = __builtin_elementwise_max(mx, mag[w]);
  }
  // the exact largest magnitude (a cross-lane max) is needed only when e
  // must fall (a magnitude with exponent field above 142 - e) or may rise
  // (every exponent field below 135 - e)
  const int erun = vs.e;
  const uint32_t lm = mx[0] > mx[1] ? mx[0] : mx[1];
  const uint32_t lim = uint32_t(143 - erun) << 7;
  const bool lower = __any(lm >= lim);
  const bool raise = !lower && !__any(lm >= (lim > (8u << 7) ? lim - (8u << 7) : 0u));
  bool moved = false;
  if (lower || raise) {
    uint32_t top = wave_umax(lm);
    if (top >= 0x7F80u) {  // Inf or NaN present: the largest finite magnitude
      uint32_t f = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = x[w] & 0x7FFFu, hi = (x[w] >> 16) & 0x7FFFu;
        f = (lo < 0x7F80u && lo > f) ? lo : f;
        f = (hi < 0x7F80u && hi > f) ? hi : f;
      }
      top = wave_umax(f);
    }
    if (top != 0) {  // an all-zero quarter leaves e alone
      const int en = 142 - int(top >> 7);  // in [-112, 142]
      vs.e = lower ? min(erun, en) : max(erun, min(en, vs.emin + 64));
      vs.emin = min(vs.emin, vs.e);
    }
    moved = true;
  }
  const int e = vs.e;
  if (!moved && e <= 112) {
    const uint32_t b = uint32_t(112 - e) << 7;
    const u16x2 bias = __builtin_bit_cast(u16x2, b | (b << 16));
    const u16x2 three = {3, 3};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const u16x2 t = __builtin_elementwise_sub_sat(mag[w], bias) << three;
      x[w] = (x[w] & 0x80008000u) | __builtin_bit_cast(uint32_t, t);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t y = x[w];
      const f32x2 f = {__builtin_amdgcn_ldexpf(__uint_as_float(y << 16), e),
                       __builtin_amdgcn_ldexpf(__uint_as_float(y & 0xFFFF0000u), e)};
      const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
      x[w] = h;
    }
  }
  const uint32_t eb = uint32_t(e + 112);
  asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(x) : "memory");
  asm volatile("ds_write_b8 %0, %1" ::"v"(word_addr + uint32_t(wave)), "v"(eb) : "memory");
}

// LDS address of this lane's 16 bytes of the wave's quarter of a slot.
__device__ __forceinline__ uint32_t quarter_addr(const char* slot, int wave, int lane) {
  return lds_addr(slot) + 4096 + uint32_t(wave * 1024 + lane * 16);
}

__device__ __forceinline__ void group_convert(const char* slot, uint32_t word_addr, int wave,
                                              int lane, int kb, int keys, VScale& vs) {
  const uint32_t a = quarter_addr(slot, wave, lane);
  u32x4 x;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(x) : "v"(a) : "memory");
  convert_quarter(x, a, word_addr, wave, lane, kb, keys, vs);
}

// What a group sub-block reads and writes beside its own operands: the
// current slot's exponent word, and the next sub-block's quarter, which the
// wave converts while it computes the current one (its LDS address, this
// lane's 16 bytes; its slot's exponent word; its first key; the wave's
// V exponent).
struct NextQuarter {
  uint32_t word_cur;
  uint32_t a, word_addr;
  int kb, wave;
  VScale* vs;
};

// How a sub-block's V operands are read and fed to the PV product.
//  kVPrivate: a single-tile item's private slot, plain LDS reads, bf16 V;
//    V past the key count is zeroed in registers (EDGE).
//  kVGroupF16: the shared ring of a group item, opaque reads; group_convert
//    has zeroed V past the key count and rewritten every d tile as fp16,
//    scaled by 2^e (e from the slot's exponent word vword); the PV and l
//    products run on the fp16 MFMA (accumulate16).
enum { kVPrivate = 0, kVGroupF16 = 1 };

// Exponent e of d tile dt in an exponent word (bytes hold e + 112).
__device__ __forceinline__ int vexp(uint32_t word, int dt) {
  return int((word >> (8 * dt)) & 0xFFu) - 112;
}

// One 32-key sub-block for QPW q tiles. The scores of every q tile come
// first, with the lane's max score of each; one wave-uniform test then says
// whether any score exceeds its column's threshold (or this is the wave's
// first sub-block), in which case every q tile rebases (rare). The weights
// and accumulation of every q tile follow the join, in place over the
// scores, so nothing is computed twice and the accumulators stay in their
// registers on both paths. EDGE: the sub-block reaches past some row's
// causal limit or past the key count, so scores are masked (and, for
// kVPrivate, V past the key count is zeroed). nxt (kVGroupF16): the slot's
// exponent word, read with the K operands (when it differs from the wave's,
// the accumulators of each d tile move to the new scale, 2^(e_new - e_old),
// exactly, on the rebase path), and the next sub-block's quarter, read with
// them too and converted before the products, so that its LDS write has
// landed by the next barrier.
template <int QPW, bool EDGE, int VMODE = kVPrivate>
__device__ __forceinline__ void sub_block(const char* sub, int kb, int keys, bool first,
                                          const u32x4 (&qop)[QPW][2], const int (&nq)[QPW],
                                          WaveState<QPW>& st, int lane, uint32_t kr0,
                                          const Consts& kc, const NextQuarter& nxt = NextQuarter{}) {
  constexpr bool OPAQUE = VMODE != kVPrivate;
  const int G = lane >> 4;
  auto rd = [&](uint32_t off) { return *reinterpret_cast<const u32x4*>(sub + off); };
  // d-step 1 flips bit 2 of the chunk index; computed here by an opaque
  // instruction so that it is not hoisted into a second live register
  uint32_t kr1;
  asm volatile("v_xor_b32 %0, 64, %1" : "=v"(kr1) : "v"(kr0));
  u32x4 k[4];
  uint32_t vword = 0;  // kVGroupF16: the slot's exponent word
  if constexpr (OPAQUE) {
    const uint32_t base = lds_addr(sub);
    u32x4 xq;
    uint32_t wv;
    lds_read_k_q(k, xq, wv, base + kr0, base + kr1, nxt.a, nxt.word_cur);
    vword = uint32_t(__builtin_amdgcn_readfirstlane(int(wv)));
    convert_quarter(xq, nxt.a, nxt.word_addr, nxt.wave, lane, nxt.kb, keys, *nxt.vs);
  } else {
    k[0] = rd(kr0);
    k[1] = rd(kr1);
    k[2] = rd(kr0 + 512);
    k[3] = rd(kr1 + 512);
  }
  float sc[QPW][8];
  bool over = false;
#pragma unroll
  for (int u = 0; u < QPW; ++u) {
    scores<QPW, EDGE>(k, qop, u, kb, G, nq, sc[u]);
    // the running max takes the sub-block's scores in four v_maximum3; the
    // threshold test reads it (scores seen before this sub-block are below
    // the threshold already: a rebase puts it above every score so far)
    st.ms[u] = max3(st.ms[u], max3(sc[u][0], sc[u][1], sc[u][2]), max3(sc[u][3], sc[u][4], sc[u][5]));
    st.ms[u] = max3(st.ms[u], sc[u][6], sc[u][7]);
    over |= st.ms[u] > st.thr[u];
  }
  bool rescale = false;
  if constexpr (VMODE == kVGroupF16) rescale = vword != st.ev;
  if (first || rescale || __any(over)) {
#pragma unroll
    for (int u = 0; u < QPW; ++u) rebase<QPW, (VMODE == kVGroupF16) ? kPShift16 : 0>(st, u, st.ms[u]);
    if constexpr (VMODE == kVGroupF16) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int de = vexp(vword, dt) - vexp(st.ev, dt);
#pragma unroll
        for (int u = 0; u < QPW; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) st.acc[dt][u][e] = __builtin_amdgcn_ldexpf(st.acc[dt][u][e], de);
      }
      st.ev = vword;
    }
  }
  // V operands only now: K is dead, so the two are never live together
  u32x4 v[4];
  if constexpr (OPAQUE) {
    lds_read_v(v, lds_addr(sub) + 4096 + lane * 16);
  } else {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) v[dt] = rd(4096 + dt * 1024 + lane * 16);
  }
  if constexpr (VMODE == kVPrivate && EDGE) {
    if (kb + 32 > keys) {  // slots past the key count may hold anything
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int w = 0; w < 4; ++w) v[dt][w] = zero_past(v[dt][w], kb + 8 * G + 2 * w, keys);
    }
  }
  if constexpr (VMODE == kVGroupF16) {
    uint32_t o16 = 0x3C003C00u;  // fp16 (1, 1), in a register (see Consts)
    asm volatile("" : "+v"(o16));
    const u32x4 ones16 = u32x4{o16, o16, o16, o16};
#pragma unroll
    for (int u = 0; u < QPW; ++u) accumulate16<QPW>(st, u, sc[u], v, ones16);
    // as below, with five MFMAs and 20 VALU instructions a q tile
    __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
#pragma unroll
    for (int i = 0; i < 5 * QPW; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
  } else {
#pragma unroll
    for (int u = 0; u < QPW; ++u) accumulate<QPW>(st, u, sc[u], v, kc);
    // Schedule: q tile 0's weights first, then every MFMA of the PV and l
    // products followed by VALU work of the later q tiles. Left alone, the
    // compiler puts all weights before all MFMAs, and the matrix core idles
    // while the wave computes weights and the other way round.
    if constexpr (QPW > 1) {
      __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);  // VALU: q tile 0
#pragma unroll
      for (int i = 0; i < 10 * QPW; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
      }
    }
  }
}

// One q tile's state as the waves fold it at the end: o accumulators, the
// exponent base, the true max and l at the base.
struct TileState {
  f32x4 acc[4];
  float mref, mtrue, l;
};

// Fold state b into a (a first, then b: the order is fixed).
__device__ __forceinline__ void fold(TileState& a, const TileState& b) {
  const float c = kScale * kLog2e;
  const float ninf = -__builtin_inff();
  const float mn = fmaxf(a.mref, b.mref);
  const float base = (mn == ninf) ? 0.f : mn;
  const float a0 = exp2_((a.mref - base) * c);
  const float a1 = exp2_((b.mref - base) * c);
  a.mref = mn;
  a.mtrue = fmaxf(a.mtrue, b.mtrue);
  a.l = __builtin_fmaf(b.l, a1, a.l * a0);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_fmaf(b.acc[dt][i], a1, a.acc[dt][i] * a0);
    a.acc[dt] = r;
  }
}

template <int QPW>
__device__ __forceinline__ TileState tile_of(const WaveState<QPW>& st, const float (&mtrue)[QPW],
                                             int u) {
  return TileState{{st.acc[0][u], st.acc[1][u], st.acc[2][u], st.acc[3][u]}, st.mref[u], mtrue[u],
                   st.l[u][0]};
}

// A published tile state in LDS: per lane 4 f32x4 of o, then mref, mtrue, l
// (lane-major arrays, so every access is one conflict-free LDS op).
constexpr int kTileFloats = 19 * 64;

__device__ __forceinline__ void put_tile(float* slot, const TileState& t, int lane) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(slot + (dt * 64 + lane) * 4) = t.acc[dt];
  slot[1024 + lane] = t.mref;
  slot[1088 + lane] = t.mtrue;
  slot[1152 + lane] = t.l;
}

__device__ __forceinline__ TileState get_tile(const float* slot, int lane) {
  TileState t;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) t.acc[dt] = *reinterpret_cast<const f32x4*>(slot + (dt * 64 + lane) * 4);
  t.mref = slot[1024 + lane];
  t.mtrue = slot[1088 + lane];
  t.l = slot[1152 + lane];
  return t;
}

// What every item reads first: its work record, then, in one round trip
// (all four depend on the work record only), its first tile, its stream's
// record and the stream's K and V addresses for the layer.
struct Item {
  asv_work wk;
  asv_tile T;
  asv_seg S;
  const uint16_t* K;
  const uint16_t* V;
};

// A block of 4 waves runs one work item; every wave holds all QPW q tiles
// of the tile (QPW = ceil(rows/4)) and its own stripe of the split's keys;
// at the end the waves fold their states through LDS in wave order.
template <int QPW, int AUX>
__device__ __forceinline__ void attn_item(const TableView& tv, const Item& it,
                                          const uint16_t* __restrict__ Q, float* __restrict__ po,
                                          float* __restrict__ pml, char* __restrict__ ringA,
                                          char* __restrict__ ringB) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = lane >> 4;
  const int c16 = lane & 15;
  const asv_work& wk = it.wk;
  const asv_tile& T = it.T;
  const asv_seg& S = it.S;
  const int g = wk.head;
  // visible key counts come from the table's rows (causal: the tile's first
  // row sees the fewest; block tables: every row sees all keys)
  const int n_first = uni(cload(tv.rows + T.row0).nkeys);
  const int k0 = split_start(S, wk.split);
  const int k1 = k0 + wk.keys;  // the split's keys the tile's last row sees
  const int64_t head_elems = int64_t(S.cap) * ASV_HEAD_DIM;
  const uint16_t* Kh = it.K + g * head_elems;
  const uint16_t* Vh = it.V + g * head_elems;

  // per-lane byte offsets: HBM chunks fetched into K group j and V group dt
  // (1 KB on per dt), and the K operands read back for d-steps 0 and 1
  uint32_t koff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) koff[j] = uint32_t(j * 1024) + k_fetch(lane, j);
  const uint32_t voff = uint32_t(c16 * 64 + G * 16);  // V^T[16dt + c16][8G .. 8G+7]
  const uint32_t kr0 = k_read(G, c16, 0);
  const Consts kc = make_consts();

  // Q operands (B of the score MFMA, held in registers for the whole item)
  // and each column's visible key count
  WaveState<QPW> st;
  u32x4 qop[QPW][2];
  int nq[QPW];
  const float ninf = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < QPW; ++u) {
    const int q = u * 16 + c16;
    const int rt = q >> 2;
    if (rt < T.nrows) {
      const uint16_t* qp =
          Q + (int64_t(T.row0 + rt) * ASV_Q_HEADS + g * 4 + (q & 3)) * ASV_HEAD_DIM + 8 * G;
      qop[u][0] = load16(qp);
      qop[u][1] = load16(qp + 32);
      nq[u] = gload(tv.rows + T.row0 + rt).nkeys;
    } else {
      qop[u][0] = u32x4{0u, 0u, 0u, 0u};
      qop[u][1] = u32x4{0u, 0u, 0u, 0u};
      nq[u] = 0;
    }
    st.mref[u] = ninf;
    st.nmc[u] = 0.f;
    st.thr[u] = ninf;
    st.ms[u] = ninf;
    st.l[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.acc[dt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  char* slotA = ringA + wave * kSubBytes;
  char* slotB = ringB + wave * kSubBytes;
  const int stride = kWaves * 32;
  const int first = k0 + wave * 32;
  const int nb = first < k1 ? (k1 - first + stride - 1) / stride : 0;

  // first ring fill after the Q loads, then retire the Q loads: the loop's
  // waits then count ring loads only
  if (nb > 0) {
    issue_sub<AUX>(slotA, Kh, Vh, first, koff, voff);
    wait_vm<8>();
  } else {
    wait_vm<0>();
  }

  // two-slot ring, one sub-block an iteration: while one slot is consumed
  // the next sub-block's 8 loads are in flight into the other. The wave's
  // sub-blocks that reach past the tile's first row's causal limit (edge
  // sub-blocks, masked) all come after the interior ones, so the two kinds
  // run in two loops, each with one copy of the sub-block code: values then
  // stay in their registers from one iteration to the next.
  auto step = [&](int i) -> const char* {
    const bool odd = (i & 1) != 0;
    if (i + 1 < nb) {
      issue_sub<AUX>(odd ? slotA : slotB, Kh, Vh, first + (i + 1) * stride, koff, voff);
      wait_vm<8>();
    } else {
      wait_vm<0>();
    }
    return odd ? slotB : slotA;
  };
  // interior: first + i * stride + 32 <= n_first
  const int lim = n_first - 32 - first;
  const int n_in = lim < 0 ? 0 : min(nb, lim / stride + 1);
  int i = 0;
  for (; i < n_in; ++i) {
    const char* cur = step(i);
    sub_block<QPW, false>(cur, first + i * stride, S.keys, i == 0, qop, nq, st, lane, kr0, kc);
  }
  for (; i < nb; ++i) {
    const char* cur = step(i);
    sub_block<QPW, true>(cur, first + i * stride, S.keys, i == 0, qop, nq, st, lane, kr0, kc);
  }
  // true maxima (the four lanes of a column saw its keys 8G..8G+7 of every
  // sub-block; the column sums are already whole)
  const float c = kScale * kLog2e;
  float mtrue[QPW];
#pragma unroll
  for (int u = 0; u < QPW; ++u) mtrue[u] = max_xor32(max_xor16(st.ms[u]));
  __syncthreads();  // the rings are reused for the fold

  // Fold: wave u (u < QPW) owns q tile u. Every wave publishes the states of
  // the tiles it does not own (at most 12 slots of 4,864 bytes: six in each
  // ring array), then wave u folds tile u over waves 0, 1, 2, 3 in that order
  // and writes its records.
  constexpr int kPer = (QPW == 4) ? 3 : QPW;  // slots a wave publishes
  auto slot = [&](int w, int u) -> float* {
    const int i = w * kPer + ((QPW == 4 && u > w) ? u - 1 : u);
    char* base = (i < 6) ? ringA : ringB;
    return reinterpret_cast<float*>(base + (i % 6) * kTileFloats * 4);
  };
  static_assert(6 * kTileFloats * 4 <= kWaves * kSubBytes, "published states fit the ring");
#pragma unroll
  for (int u = 0; u < QPW; ++u)
    if (u != wave) put_tile(slot(wave, u), tile_of(st, mtrue, u), lane);
  __syncthreads();
  if (wave >= QPW) return;
  const int u = wave;
  TileState own;
#pragma unroll
  for (int t = 0; t < QPW; ++t)
    if (t == u) own = tile_of(st, mtrue, t);
  TileState a = (u == 0) ? own : get_tile(slot(0, u), lane);
  for (int w = 1; w < kWaves; ++w) fold(a, (w == u) ? own : get_tile(slot(w, u), lane));

  // records: o = acc / l (any exponent base), then (true max in score units,
  // l taken to the true max)
  const int q = u * 16 + c16;
  const int rt = q >> 2;
  if (rt >= T.nrows) return;
  const int64_t rec =
      S.poff + (int64_t(wk.split) * S.rows + T.pos0 + rt) * ASV_Q_HEADS + g * 4 + (q & 3);
  const float L = a.l;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (L > 0.f) ? a.acc[dt][i] / L : 0.f;
    store16f(po + rec * ASV_HEAD_DIM + dt * 16 + 4 * G, r);
  }
  if (G == 0) {
    const float mt = a.mtrue;
    const float lt = (mt == ninf) ? 0.f : L * exp2_((a.mref - mt) * c);
    gstore(reinterpret_cast<float2*>(pml) + rec, make_float2((mt == ninf) ? ninf : mt * kScale, lt));
  }
}

// Group items (ntiles > 1): up to four consecutive 16-row tiles of one
// multi-tile stream (a prompt chunk) and one split. Wave w owns tile w of
// the group, all four of its q tiles, and walks every sub-block of the
// split; the four waves share one ring of kGroupSlots sub-blocks, each wave
// filling a quarter of every sub-block (K group w and V group w, 2 KB), with
// one block barrier a sub-block. Each K/V byte so enters LDS once for up to
// four tiles where single-tile items fetch it once a tile, which cuts the
// L2 requests of chunks fourfold, and there is no fold between waves.
constexpr int kGroupSlots = 8;  // 64 KB: both ring arrays

// Block barrier of the shared ring. __syncthreads() would also wait for
// every LDS write the wave has in flight, the ring's direct loads included
// (vmcnt(0)), which would drain the ring at every sub-block; the loads that
// must have landed are waited for explicitly before this. The empty asm
// statements keep the compiler from moving memory accesses across it, and
// lgkmcnt(0) retires the wave's LDS reads of the slot about to be refilled.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt: no wait
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int AUX>
__device__ __forceinline__ void issue_quarter(char* slot, const uint16_t* __restrict__ Kh,
                                              const uint16_t* __restrict__ Vh, int kb,
                                              uint32_t koff, uint32_t voff, int wave) {
  const char* kbase = reinterpret_cast<const char*>(Kh + int64_t(kb) * ASV_HEAD_DIM);
  const char* vbase =
      reinterpret_cast<const char*>(Vh + int64_t(kb >> 5) * (ASV_HEAD_DIM * 32)) + wave * 1024;
  lds_dma16<AUX>(kbase, koff, slot + wave * 1024);
  lds_dma16<AUX>(vbase, voff, slot + 4096 + wave * 1024);
}

template <int AUX>
__device__ __forceinline__ void attn_group(const TableView& tv, const Item& it,
                                           const uint16_t* __restrict__ Q, float* __restrict__ po,
                                           float* __restrict__ pml, char* __restrict__ ringA,
                                           char* __restrict__ ringB, uint32_t* __restrict__ vword) {
  constexpr int QPW = 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = lane >> 4;
  const int c16 = lane & 15;
  const asv_work& wk = it.wk;
  const bool active = wave < wk.ntiles;
  const asv_tile& T0 = it.T;
  const asv_tile T = uniform(cload(tv.tiles + wk.tile + (active ? wave : 0)));
  const asv_seg& S = it.S;
  const int g = wk.head;
  // the group's first row sees the fewest keys
  const int n_first = uni(cload(tv.rows + T0.row0).nkeys);
  const int k0 = split_start(S, wk.split);
  const int k1 = k0 + wk.keys;  // the split's keys the group's last row sees
  const int64_t head_elems = int64_t(S.cap) * ASV_HEAD_DIM;
  const uint16_t* Kh = it.K + g * head_elems;
  const uint16_t* Vh = it.V + g * head_elems;

  // this wave's quarter of each sub-block: K group `wave`, V group `wave`
  const uint32_t koff = uint32_t(wave * 1024) + k_fetch(lane, wave);
  const uint32_t voff = uint32_t(c16 * 64 + G * 16);
  const uint32_t kr0 = k_read(G, c16, 0);
  const Consts kc = make_consts();

  WaveState<QPW> st;
  st.ev = 0x70707070u;  // e = 0 (the first sub-block takes the rebase path)
  u32x4 qop[QPW][2];
  int nq[QPW];
  const float ninf = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < QPW; ++u) {
    const int q = u * 16 + c16;
    const int rt = q >> 2;
    if (active && rt < T.nrows) {
      const uint16_t* qp =
          Q + (int64_t(T.row0 + rt) * ASV_Q_HEADS + g * 4 + (q & 3)) * ASV_HEAD_DIM + 8 * G;
      qop[u][0] = load16(qp);
      qop[u][1] = load16(qp + 32);
      nq[u] = gload(tv.rows + T.row0 + rt).nkeys;
    } else {
      qop[u][0] = u32x4{0u, 0u, 0u, 0u};
      qop[u][1] = u32x4{0u, 0u, 0u, 0u};
      nq[u] = 0;
    }
    st.mref[u] = ninf;
    st.nmc[u] = 0.f;
    st.thr[u] = ninf;
    st.ms[u] = ninf;
    st.l[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.acc[dt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto slot = [&](int s) -> char* {
    return ((s & 4) ? ringB : ringA) + (s & 3) * kSubBytes;
  };
  const int nb = (k1 - k0 + 31) >> 5;  // >= 1: an item exists only for visible keys
  // prologue: the first kGroupSlots - 1 sub-blocks in flight. Always as
  // many loads (a split of fewer sub-blocks re-reads its last one into the
  // spare slots), so that the wait below retires the Q loads on every path
  // and the compiler adds no wait of its own for them inside the loop.
#pragma unroll
  for (int s = 0; s < kGroupSlots - 1; ++s)
    issue_quarter<AUX>(slot(s), Kh, Vh, k0 + 32 * min(s, nb - 1), koff, voff, wave);
  wait_vm<2 * (kGroupSlots - 2)>();

  // Iteration i: this wave's loads of sub-block i have landed (older loads
  // retire first), then the barrier says every wave's have, and that every
  // wave is done with sub-block i - 1, whose slot is refilled with sub-block
  // i + kGroupSlots - 1 before sub-block i is computed.
  const uint32_t word0 = lds_addr(reinterpret_cast<const char*>(vword));
  VScale vsc;  // this wave's V exponent (d tile `wave`)
  // sub-block 0's quarter now; sub-block i + 1's while sub-block i is
  // computed (its loads have landed before barrier i)
  group_convert(slot(0), word0, wave, lane, k0, S.keys, vsc);
  auto step = [&](int i) -> const char* {
    if (i + kGroupSlots - 2 < nb) wait_vm<2 * (kGroupSlots - 3)>();
    else wait_vm<0>();
    const int s = i & (kGroupSlots - 1);
    ring_barrier();
    const int nx = i + kGroupSlots - 1;
    if (nx < nb) issue_quarter<AUX>(slot(nx & (kGroupSlots - 1)), Kh, Vh, k0 + 32 * nx, koff, voff, wave);
    return slot(s);
  };
  // sub-block i of the slot just returned by step(i), with its exponent
  // word; the quarter of sub-block i + 1 is converted meanwhile (after the
  // last sub-block that is a spare slot with no load in flight: the
  // conversion is harmless there)
  auto run = [&](auto edge, const char* cur, int i) {
    constexpr bool E = decltype(edge)::value;
    const int sn = (i + 1) & (kGroupSlots - 1);
    const NextQuarter nxt{word0 + 4 * uint32_t(i & (kGroupSlots - 1)),
                          quarter_addr(slot(sn), wave, lane), word0 + 4 * sn, k0 + 32 * (i + 1),
                          wave, &vsc};
    if (active) {
      sub_block<QPW, E, kVGroupF16>(cur, k0 + 32 * i, S.keys, i == 0, qop, nq, st, lane, kr0, kc,
                                    nxt);
    } else {
      group_convert(slot(sn), nxt.word_addr, wave, lane, nxt.kb, S.keys, vsc);
    }
  };
  // interior sub-blocks: every row of the group sees all of their keys
  const int lim = n_first - 32 - k0;
  const int n_in = lim < 0 ? 0 : min(nb, lim / 32 + 1);
  int i = 0;
  for (; i < n_in; ++i) {
    const char* cur = step(i);
    run(std::false_type{}, cur, i);
  }
  for (; i < nb; ++i) {
    const char* cur = step(i);
    run(std::true_type{}, cur, i);
  }
  if (!active) return;

  // records of the wave's own tile: o = acc / l, then (true max in score
  // units, l taken to the true max)
  const float c = kScale * kLog2e;
#pragma unroll
  for (int u = 0; u < QPW; ++u) {
    const float L = st.l[u][0];
    const float mt = max_xor32(max_xor16(st.ms[u]));
    const int q = u * 16 + c16;
    const int rt = q >> 2;
    if (rt < T.nrows) {
      const int64_t rec =
          S.poff + (int64_t(wk.split) * S.rows + T.pos0 + rt) * ASV_Q_HEADS + g * 4 + (q & 3);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        f32x4 r;
        const int ed = -vexp(st.ev, dt);  // back from the scale of d tile dt
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r[e] = (L > 0.f) ? __builtin_amdgcn_ldexpf(st.acc[dt][u][e] / L, ed) : 0.f;
        store16f(po + rec * ASV_HEAD_DIM + dt * 16 + 4 * G, r);
      }
      if (G == 0) {
        const float lt =
            (mt == ninf) ? 0.f : __builtin_amdgcn_ldexpf(L, -kPShift16) * exp2_((st.mref[u] - mt) * c);
        gstore(reinterpret_cast<float2*>(pml) + rec, make_float2((mt == ninf) ? ninf : mt * kScale, lt));
      }
    }
  }
}

template <int QPW_MAX>
__global__ __launch_bounds__(kThreads, 2) void attn_split(TableView tv, int layer,
                                                          const uint16_t* __restrict__ Q,
                                                          float* __restrict__ po,
                                                          float* __restrict__ pml) {
  // two ring slots per wave, as two arrays so the compiler can tell a slot
  // being loaded from the one being read; the fold reuses them afterwards
  __shared__ __attribute__((aligned(16))) char ringA[kWaves * kSubBytes];
  __shared__ __attribute__((aligned(16))) char ringB[kWaves * kSubBytes];
  __shared__ uint32_t vword[kGroupSlots];  // group items: V exponents a slot
  Item it;
  it.wk = uniform(cload(tv.work + blockIdx.x));
  const asv_work& wk = it.wk;
  it.T = uniform(cload(tv.tiles + wk.tile));
  it.S = uniform(cload(tv.segs + wk.stream));
  const int64_t sel = int64_t(layer) * tv.n_streams + wk.stream;
  it.K = reinterpret_cast<const uint16_t*>(uniform_ptr(cload(tv.kp + sel)));
  it.V = reinterpret_cast<const uint16_t*>(uniform_ptr(cload(tv.vp + sel)));
  // no instruction moves across this point, so the four reads above are all
  // issued before the first wait for any of them
  __builtin_amdgcn_sched_barrier(0);
  const asv_tile& T = it.T;
  const int nqt = (T.nrows + 3) >> 2;
  // an item that covers every tile of its stream reads its K/V once: stream
  // it past the caches; items of a longer stream re-read the same keys
  const bool once = T.pos0 == 0 && it.S.rows <= ASV_TILE_ROWS * int(wk.ntiles);
  if constexpr (QPW_MAX >= 4) {
    // groups come only from streams of more than one tile, whose tiles
    // (the last aside) hold 16 rows, so a round that has them launches this
    // instance
    if (wk.ntiles > 1) {
      if (once) return attn_group<kStream>(tv, it, Q, po, pml, ringA, ringB, vword);
      return attn_group<0>(tv, it, Q, po, pml, ringA, ringB, vword);
    }
    if (nqt == 4) {
      if (once) return attn_item<4, kStream>(tv, it, Q, po, pml, ringA, ringB);
      return attn_item<4, 0>(tv, it, Q, po, pml, ringA, ringB);
    }
  }
  if constexpr (QPW_MAX >= 3) {
    if (nqt == 3) {
      if (once) return attn_item<3, kStream>(tv, it, Q, po, pml, ringA, ringB);
      return attn_item<3, 0>(tv, it, Q, po, pml, ringA, ringB);
    }
  }
  if constexpr (QPW_MAX >= 2) {
    if (nqt == 2) {
      if (once) return attn_item<2, kStream>(tv, it, Q, po, pml, ringA, ringB);
      return attn_item<2, 0>(tv, it, Q, po, pml, ringA, ringB);
    }
  }
  if (once) return attn_item<1, kStream>(tv, it, Q, po, pml, ringA, ringB);
  attn_item<1, 0>(tv, it, Q, po, pml, ringA, ringB);
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

