// Markov-head step of the drafter: each drafted row's pick from its logits
// plus W2 . W1[previous token] (gfx950).
//
// PR #1391 "lfm2: draft with LiquidAI's DSpark drafter (--drafter)",
// description and new-kernel list: the drafter's Markov head scores a block
// row as its logits plus W2 . W1[token before the row] and takes that row's
// argmax before the next row, which uses the pick as its previous token
// (lowest token on a tie, a NaN score flagged); its testing notes write the
// score as
// bf16(base + bf16(W2 . W1[prev])), at rows x vocabulary x rank
// 1 x 128,000 x 256; the config admission caps the rank at 256. The exact
// arithmetic (float32 dot, k ascending, one rounding per term) is written
// out in include/asv_draft.h.
//
// Two forms of a pass, the same bits from either: a resident form (one
// launch for the whole pass, W2 kept in registers; further below, where its
// kernel is) taken whenever its blocks fit on the device at once, and the
// form described here, one launch a depth.
//
// A pass of depth D is D scan launches and one fold launch, no atomics.
// The scan of depth j scores every chain's row at that depth and leaves,
// per chain, one 4-byte record a block (its best order key and lane, and a
// nonfinite bit). The scan of depth j + 1 starts by folding those records
// in every block (each block needs the previous tokens; the records are a
// few KB and are read from cache, while the block's W2 loads, issued right
// after them, stream from HBM), and its block 0 writes depth j's picks and
// flags. A last one-block launch folds the deepest depth. Depths alternate
// between the two halves of the workspace, so no block overwrites records
// that another block of the same launch still folds.
//
// Scan: one thread per token v, 256 tokens a block. W2 is stored in tiles
// of 64 tokens (one wave's), each [rank/8][64][8]: the 8 coefficients
// k = 8c..8c+7 of the tile's tokens at chunk c, so one 16-byte load per lane
// per chunk is a contiguous 1 KB, and a wave's rank/8 loads are one
// contiguous run of rank * 128 bytes (faster than chunks a whole vocabulary
// apart). A lane holds all rank/8 chunks of its token (up to 128 VGPRs,
// 32 KB a wave in flight), requested in two halves with the chains' W1
// pieces between them, so the W1 rows are ready while the second half
// still streams. The chains' W1 rows are the same for the whole block:
// they are converted to float32 into LDS once, and each
// multiply-add reads its W1 value by an LDS broadcast. The dot is summed one
// k at a time in float32 (a fused multiply-add of an exact product), four
// chains at a time so that each converted W2 value serves four chains.

#include <array>
#include <atomic>
#include <climits>
#include <utility>

#include "device.h"
#include "asv_draft.h"

namespace asv {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChains = ASV_MARKOV_MAX_CHAINS;
constexpr int kMaxChunks = ASV_MARKOV_MAX_RANK / 8;
constexpr int kGroup = 4;  // chains scored together

// One depth: the chains scored at it, and the chains of the depth before,
// whose block records the launch folds first.
struct Step {
  int32_t n;                  // chains scored at this depth
  int32_t row[kMaxChains];    // chain i's logits / pick row
  int32_t src[kMaxChains];    // its previous token: src >= 0, the fold result of
                              // chain src of the depth before; src < 0, prev0[-1 - src]
  int32_t nprev;              // chains of the depth before (0 at the first depth)
  int32_t prow[kMaxChains];   // their pick rows
};

// Order key of a non-NaN bf16 pattern: larger key = larger value; -0 and +0
// share a key. Every non-NaN pattern has a key >= 0x7F.
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  b = (b == 0x8000u) ? 0u : b;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}

__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  x = umax_xor32(x);
  x = umax_xor16(x);
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    const uint32_t o = uint32_t(__shfl_xor(int(x), off));
    x = o > x ? o : x;
  }
  return x;
}

// A block record of a block of THREADS threads (LB = log2 THREADS bits of
// lane): bits LB..LB+15 the order key of the block's largest score and bits
// 0..LB-1 THREADS - 1 - its thread (so the lower token wins a tie inside the
// block), both 0 when every score of the block is NaN; bit 31 the nonfinite
// flag.
template <int THREADS>
struct RecBits {
  static constexpr int kLB = __builtin_ctz(THREADS);
  static_assert((1 << kLB) == THREADS && kLB + 16 <= 31, "a power of two below 2^15");
  static constexpr uint32_t kKey = (1u << (kLB + 16)) - 1u;
  static constexpr uint32_t kLane = THREADS - 1u;
};
constexpr uint32_t kRecBad = 0x80000000u;

// Fold one chain's records (nblocks of them) in one wave: the largest order
// key, then the lowest token. Loads are issued by fold_load (eight a lane in
// flight) and consumed by fold_use, so a caller can put other loads after
// them.
struct FoldAcc {
  uint32_t hi, lo;  // (order key, ~token) of the best so far, (0, 0) for none
  bool bad;
};

template <int THREADS>
__device__ __forceinline__ void fold_use(FoldAcc& a, const uint32_t (&e)[8], int b0, int lane) {
  using R = RecBits<THREADS>;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t key = e[u] & R::kKey;
    a.bad |= (e[u] & kRecBad) != 0u;
    if (key != 0u) {
      const uint32_t b = uint32_t(b0 + u * 64 + lane);
      const uint32_t tok = b * THREADS + (R::kLane - (key & R::kLane));
      const uint32_t hi = key >> R::kLB, lo = ~tok;
      if (hi > a.hi || (hi == a.hi && lo > a.lo)) {
        a.hi = hi;
        a.lo = lo;
      }
    }
  }
}

__device__ __forceinline__ void fold_load(uint32_t (&e)[8], const uint32_t* __restrict__ rec, int nblocks,
                                          int b0, int lane) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int b = b0 + u * 64 + lane;
    e[u] = b < nblocks ? gload(rec + b) : 0u;
  }
}

// Wave-wide result of a fold: the token (0 when every score was NaN) and the flag.
__device__ __forceinline__ void fold_finish(FoldAcc a, uint32_t& tok, bool& bad) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t oh = uint32_t(__shfl_xor(int(a.hi), off));
    const uint32_t ol = uint32_t(__shfl_xor(int(a.lo), off));
    if (oh > a.hi || (oh == a.hi && ol > a.lo)) {
      a.hi = oh;
      a.lo = ol;
    }
  }
  tok = a.hi != 0u ? ~a.lo : 0u;
  bad = __any(a.bad);
}

// One depth's scores for the thread's token v: chains 0..n-1 of the depth
// (chain i's logits row row_of(i), its previous token s_prev[i]), four at a
// time so that each converted W2 value serves four chains. For chain i it
// leaves the wave's best record (the block-record layout, without the flag)
// in s_key[wave][i] and the wave's nonfinite-or-invalid flag in
// s_bad[wave][i]. w holds the token's rank/8 W2 chunks; s_w1[i] chain i's W1
// row in float32.
template <int NCH, int THREADS, class RowOf>
__device__ __forceinline__ void score_depth(int n, RowOf row_of, const int32_t* s_prev, u32x4 (&w)[NCH],
                                            const float (*s_w1)[NCH * 8], uint32_t (*s_key)[kMaxChains],
                                            uint32_t (*s_bad)[kMaxChains], const uint16_t* __restrict__ base,
                                            int64_t stride, int vc, bool live, int vocab, int tid) {
  using R = RecBits<THREADS>;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int g = 0; g < n; g += kGroup) {
    bool ok[kGroup];
    uint32_t bv[kGroup];
    int cs[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      cs[i] = min(g + i, n - 1);
      const int p = s_prev[cs[i]];
      ok[i] = p >= 0 && p < vocab;
      // unconditional (a lane past the vocabulary reads the last token and
      // is not scored), so no branch makes the compiler wait for it early
      bv[i] = uint32_t(gload(base + int64_t(row_of(cs[i])) * stride + vc));
    }

    float acc[kGroup] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      // Keep W2 as raw bf16 pairs between groups (128 VGPRs): converting it
      // once for every group would hold 256 floats and spill. The pin sits
      // at each chunk's use, so chunk c waits for its own load only and the
      // first chunks are scored while the later ones stream in.
      asm volatile("" : "+v"(w[c]));
      float f[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f[2 * k] = bf16_lo(w[c][k]);
        f[2 * k + 1] = bf16_hi(w[c][k]);
      }
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const float4 a = *reinterpret_cast<const float4*>(&s_w1[cs[i]][c * 8]);
        const float4 b = *reinterpret_cast<const float4*>(&s_w1[cs[i]][c * 8 + 4]);
        acc[i] = __builtin_fmaf(f[0], a.x, acc[i]);
        acc[i] = __builtin_fmaf(f[1], a.y, acc[i]);
        acc[i] = __builtin_fmaf(f[2], a.z, acc[i]);
        acc[i] = __builtin_fmaf(f[3], a.w, acc[i]);
        acc[i] = __builtin_fmaf(f[4], b.x, acc[i]);
        acc[i] = __builtin_fmaf(f[5], b.y, acc[i]);
        acc[i] = __builtin_fmaf(f[6], b.z, acc[i]);
        acc[i] = __builtin_fmaf(f[7], b.w, acc[i]);
      }
    }

    // The sums are pinned here, so the compiler cannot sink each chain's
    // sum into the branch that uses it (which would split the shared loop);
    // a slot past the last chain repeats it and is not stored.
#pragma unroll
    for (int i = 0; i < kGroup; ++i) asm volatile("" : "+v"(acc[i]));
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const uint32_t d = ok[i] ? f32_to_bf16(acc[i]) : 0u;
      const uint32_t s = f32_to_bf16(bf16_to_f32(uint16_t(bv[i])) + __uint_as_float(d << 16));
      const bool nonfinite = live && (s & 0x7F80u) == 0x7F80u;
      const bool nan = (s & 0x7F80u) == 0x7F80u && (s & 0x7Fu) != 0u;
      uint32_t key = (live && !nan) ? (order_key(s) << R::kLB) | uint32_t(THREADS - 1 - tid) : 0u;
      key = wave_umax(key);
      const bool bad = __any(nonfinite) || !ok[i];
      if (lane == 0 && g + i < n) {
        s_key[wave][g + i] = key;
        s_bad[wave][g + i] = bad ? 1u : 0u;
      }
    }
  }
}

// NCH = rank / 8, a compile-time count so that every chunk loop is straight
// code with no per-chunk guard.
template <int NCH>
__global__ __launch_bounds__(kThreads, 2) void markov_scan(Step st, const uint16_t* __restrict__ base,
                                                           int64_t stride, const int32_t* __restrict__ prev0,
                                                           const uint16_t* __restrict__ w1,
                                                           const uint16_t* __restrict__ w2c, int vocab,
                                                           int nblocks, const uint32_t* __restrict__ prec,
                                                           uint32_t* __restrict__ rec,
                                                           int32_t* __restrict__ pick,
                                                           uint8_t* __restrict__ flag) {
  constexpr int rank = NCH * 8;
  __shared__ __attribute__((aligned(16))) float s_w1[kMaxChains][rank];
  __shared__ uint32_t s_key[kThreads / 64][kMaxChains];
  __shared__ uint32_t s_bad[kThreads / 64][kMaxChains];
  __shared__ int32_t s_ptok[kMaxChains];
  __shared__ int32_t s_prev[kMaxChains];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int v = blockIdx.x * kThreads + tid;
  const bool live = v < vocab;
  const int vc = live ? v : vocab - 1;

  // Thread i < n's source, read with wave-uniform indexes (scalar loads of
  // the kernel argument), and at the first depth its previous token from
  // prev0: both requested before the W2 loads, since vector loads retire in
  // order and a later wait for them would wait for W2 too.
  int my_src = 0;
#pragma unroll
  for (int i = 0; i < kMaxChains; ++i)
    if (i == tid) my_src = st.src[i];
  int my_prev = 0;
  if (tid < st.n && my_src < 0) my_prev = gload(prev0 + (-1 - my_src));

  // The depth before: wave w folds its chains w, w + 4, ...; the first
  // chain's records are requested before the W2 loads, so waiting for them
  // does not wait for W2.
  const int nfold = st.nprev;
  FoldAcc fa{0u, 0u, false};
  uint32_t fe[8];
  const bool fold_first = wave < nfold;
  if (fold_first) fold_load(fe, prec + int64_t(wave) * nblocks, nblocks, 0, lane);
  __builtin_amdgcn_sched_barrier(0);

  // W2 in two halves: the first now, the second after the W1 loads, so
  // that waiting for W1 waits for the first half only and the first half
  // is scored while the second streams in (load counts retire in order)
  constexpr int kHalf = (NCH + 1) / 2;
  u32x4 w[NCH];
  // the wave's 64-token tile of W2: chunk c of its tokens at c * tl * 8 from
  // the tile's start, tl = the tile's token count (64 but in the last tile)
  const int64_t tile = vc / 64;
  const int64_t tl = min(int64_t(64), int64_t(vocab) - tile * 64);
  const uint16_t* wp = w2c + tile * 64 * rank + (vc - tile * 64) * 8;
  const int64_t plane = tl * 8;
#pragma unroll
  for (int c = 0; c < kHalf; ++c) w[c] = load16(wp + c * plane);
  __builtin_amdgcn_sched_barrier(0);

  // chain ci's fold result: its previous token for this block, and block 0
  // writes it as the depth before's pick
  auto fold_done = [&](int ci, FoldAcc a) {
    uint32_t tok;
    bool bad;
    fold_finish(a, tok, bad);
    if (lane == 0) {
      s_ptok[ci] = int32_t(tok);
      if (blockIdx.x == 0) {
        // ci is wave-uniform: a scalar read of the row, not a vector load
        // whose wait would wait for the W2 loads in flight
        const int pr = st.prow[__builtin_amdgcn_readfirstlane(ci)];
        gstore(pick + pr, int32_t(tok));
        gstore(flag + pr, uint8_t(bad ? 1 : 0));
      }
    }
  };
  // The first chain apart from the loop below, so that its wait (on the
  // records only) is not merged with the reloads' waits (on everything).
  if (fold_first) {
    fold_use<kThreads>(fa, fe, 0, lane);
    for (int b0 = 64 * 8; b0 < nblocks; b0 += 64 * 8) {
      fold_load(fe, prec + int64_t(wave) * nblocks, nblocks, b0, lane);
      fold_use<kThreads>(fa, fe, b0, lane);
    }
    fold_done(wave, fa);
  }
  for (int ci = wave + kThreads / 64; ci < nfold; ci += kThreads / 64) {
    const uint32_t* r = prec + int64_t(ci) * nblocks;
    FoldAcc a{0u, 0u, false};
    for (int b0 = 0; b0 < nblocks; b0 += 64 * 8) {
      fold_load(fe, r, nblocks, b0, lane);
      fold_use<kThreads>(a, fe, b0, lane);
    }
    fold_done(ci, a);
  }
  __syncthreads();

  // previous tokens, then the chains' W1 rows in float32 (row 0 stands in
  // for an invalid token: its sum is replaced by +0)
  if (tid < st.n) s_prev[tid] = my_src >= 0 ? s_ptok[my_src] : my_prev;
  __syncthreads();
  // one 16-byte piece of a W1 row a thread and pass (n * rank / 8 pieces,
  // at most 1,024: four passes), all requested before the second W2 half
  constexpr int kPass = (kMaxChains * NCH + kThreads - 1) / kThreads;
  u32x4 q[kPass];
#pragma unroll
  for (int k = 0; k < kPass; ++k) {
    const int idx = tid + k * kThreads;
    if (idx < st.n * NCH) {
      const int ci = idx / NCH;
      const int p = s_prev[ci];
      const bool ok = p >= 0 && p < vocab;
      q[k] = load16(w1 + int64_t(ok ? p : 0) * rank + (idx - ci * NCH) * 8);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = kHalf; c < NCH; ++c) w[c] = load16(wp + c * plane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < kPass; ++k) {
    const int idx = tid + k * kThreads;
    if (idx < st.n * NCH) {
      const int ci = idx / NCH;
      const int c = idx - ci * NCH;
      float4 a, b;
      a.x = bf16_lo(q[k][0]); a.y = bf16_hi(q[k][0]); a.z = bf16_lo(q[k][1]); a.w = bf16_hi(q[k][1]);
      b.x = bf16_lo(q[k][2]); b.y = bf16_hi(q[k][2]); b.z = bf16_lo(q[k][3]); b.w = bf16_hi(q[k][3]);
      *reinterpret_cast<float4*>(&s_w1[ci][c * 8]) = a;
      *reinterpret_cast<float4*>(&s_w1[ci][c * 8 + 4]) = b;
    }
  }
  __syncthreads();

  score_depth<NCH, kThreads>(st.n, [&](int i) { return st.row[i]; }, s_prev, w, s_w1, s_key, s_bad, base,
                            stride, vc, live, vocab, tid);
  __syncthreads();
  if (tid < st.n) {
    uint32_t key = 0, bad = 0;
#pragma unroll
    for (int wv = 0; wv < kThreads / 64; ++wv) {
      key = s_key[wv][tid] > key ? s_key[wv][tid] : key;
      bad |= s_bad[wv][tid];
    }
    gstore(rec + int64_t(tid) * nblocks + blockIdx.x, key | (bad ? kRecBad : 0u));
  }
}

// The deepest depth's fold, one block: wave w folds chains w, w + 4, ...
__global__ __launch_bounds__(kThreads) void markov_fold(Step st, int nblocks,
                                                        const uint32_t* __restrict__ prec,
                                                        int32_t* __restrict__ pick,
                                                        uint8_t* __restrict__ flag) {
  const int lane = threadIdx.x & 63;
  for (int ci = threadIdx.x >> 6; ci < st.nprev; ci += kThreads / 64) {
    const uint32_t* r = prec + int64_t(ci) * nblocks;
    FoldAcc fa{0u, 0u, false};
    for (int b0 = 0; b0 < nblocks; b0 += 64 * 8) {
      uint32_t e[8];
      fold_load(e, r, nblocks, b0, lane);
      fold_use<kThreads>(fa, e, b0, lane);
    }
    uint32_t tok;
    bool bad;
    fold_finish(fa, tok, bad);
    if (lane == 0) {
      gstore(pick + st.prow[ci], int32_t(tok));
      gstore(flag + st.prow[ci], uint8_t(bad ? 1 : 0));
    }
  }
}

// ---------------------------------------------------------------------------
// Resident form: the whole pass in one launch whose blocks all run at once,
// each wave holding its 64-token tile of W2 in registers from the first
// depth to the last, so W2 is read from HBM once a pass instead of once a
// depth. Between depths the blocks exchange their records through the
// workspace: a record is one 64-bit word whose upper half is its depth + 1,
// written with a single device-scope store, so a block that reads the tag
// it waits for has read that depth's record, with no other ordering
// needed; the reader polls until every block's record carries the tag. The
// records of one depth lie in the half of the workspace the next depth does
// not write (depths alternate), and a block writes depth j + 2 only after it
// read every block's depth j + 1, which each block wrote after it finished
// reading depth j; so no record is overwritten while a block still waits
// for it. The workspace is cleared by a small launch before each pass, so
// no tag left by an earlier pass is taken for one of this pass. The
// arithmetic is score_depth's, bit for bit the one-launch-a-depth form's.
//
// The launch is an ordinary one: the host admits the form only when every
// block fits on the device at once (at rank 256 one 512-thread block a CU),
// so on a device running nothing else all blocks start together; callers
// run one resident pass at a time on a device. Other work on the device can
// hold some blocks back; the others then wait, and a wait longer than
// kWaitTicks abandons the pass (flag 2 from that depth on). A
// cooperative launch would guarantee residency, but on this runtime it
// waits on the host for the stream's earlier work and costs 15-20 us a
// call on the device (measured: 112 against 93 us a pass).

constexpr int kRThreads = 512;  // 8 waves, one block a CU (the W2 tiles take 128 VGPRs a lane)
constexpr int kRWaves = kRThreads / 64;
constexpr int kRMaxBlocks = 512;  // a fold reads at most 8 records a lane

struct Chains {
  int32_t n;          // chains
  int32_t max_depth;  // the deepest chain's depth
  int32_t row0[kMaxChains];
  int32_t depth[kMaxChains];
};

// Chain c's records of one depth in one wave: polled until every block's
// carries the tag, then folded. False when wait_ticks of the 100 MHz clock
// passed with some record still missing (the pass is then abandoned).
__device__ __forceinline__ bool fold_poll(const unsigned long long* __restrict__ rec, int nblocks,
                                          uint32_t tag, int lane, uint64_t wait_ticks, uint32_t& tok,
                                          bool& bad) {
  uint32_t e[8];
  uint64_t t0 = 0;
  for (bool first = true;; first = false) {
    // all eight loads in flight together (a lane past the last block reads
    // the last block's record again), then the tests
    unsigned long long x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      x[u] = __hip_atomic_load(rec + min(u * 64 + lane, nblocks - 1), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    bool ok = true;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      ok &= uint32_t(x[u] >> 32) == tag;
      e[u] = u * 64 + lane < nblocks ? uint32_t(x[u]) : 0u;
    }
    if (__all(ok)) break;
    const uint64_t now = __builtin_amdgcn_s_memrealtime();
    if (first) t0 = now;
    else if (now - t0 > wait_ticks) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  FoldAcc a{0u, 0u, false};
  fold_use<kRThreads>(a, e, 0, lane);
  fold_finish(a, tok, bad);
  return true;
}

template <int NCH>
__global__ __launch_bounds__(kRThreads, 1) void markov_resident(
    Chains ch, const uint16_t* __restrict__ base, int64_t stride, const int32_t* __restrict__ prev0,
    const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w2c, int vocab, int nblocks,
    unsigned long long* __restrict__ rec, int32_t* __restrict__ pick, uint8_t* __restrict__ flag,
    uint64_t wait_ticks) {
  constexpr int rank = NCH * 8;
  __shared__ __attribute__((aligned(16))) float s_w1[kMaxChains][rank];
  __shared__ uint32_t s_key[kRWaves][kMaxChains];
  __shared__ uint32_t s_bad[kRWaves][kMaxChains];
  __shared__ int32_t s_tok[kMaxChains];    // chain c's previous token
  __shared__ int32_t s_row[kMaxChains];    // the depth's i-th chain: its row,
  __shared__ int32_t s_prev[kMaxChains];   // its previous token
  __shared__ int32_t s_chain[kMaxChains];  // and its chain
  __shared__ int32_t s_fail;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int v = blockIdx.x * kRThreads + tid;
  const bool live = v < vocab;
  const int vc = live ? v : vocab - 1;
  const size_t half = size_t(kMaxChains) * nblocks;

  // W1 rows of the depth's chains in float32 into LDS (row 0 stands in for
  // an invalid token): piece idx = tid + k * kRThreads is chunk idx % NCH of
  // the row of the depth's chain idx / NCH; loads first, then conversions
  constexpr int kRPass = (kMaxChains * NCH + kRThreads - 1) / kRThreads;
  auto w1_load = [&](u32x4(&q)[kRPass], int n, auto prev_of) {
#pragma unroll
    for (int k = 0; k < kRPass; ++k) {
      // unconditional (a piece past the last repeats it), so that no branch
      // makes the compiler wait for the load at once
      const int idx = min(tid + k * kRThreads, n * NCH - 1);
      const int i = idx / NCH;
      const int p = prev_of(k, i);
      const bool ok = p >= 0 && p < vocab;
      q[k] = load16(w1 + int64_t(ok ? p : 0) * rank + (idx - i * NCH) * 8);
    }
  };
  auto w1_store = [&](const u32x4(&q)[kRPass], int n) {
#pragma unroll
    for (int k = 0; k < kRPass; ++k) {
      const int idx = tid + k * kRThreads;
      if (idx < n * NCH) {
        const int i = idx / NCH;
        const int c = idx - i * NCH;
        float4 a, b;
        a.x = bf16_lo(q[k][0]); a.y = bf16_hi(q[k][0]); a.z = bf16_lo(q[k][1]); a.w = bf16_hi(q[k][1]);
        b.x = bf16_lo(q[k][2]); b.y = bf16_hi(q[k][2]); b.z = bf16_lo(q[k][3]); b.w = bf16_hi(q[k][3]);
        *reinterpret_cast<float4*>(&s_w1[i][c * 8]) = a;
        *reinterpret_cast<float4*>(&s_w1[i][c * 8 + 4]) = b;
      }
    }
  };

  // Depth 0 scores every chain, in chain order. Its previous tokens (one
  // round trip) and then its W1 rows are requested before W2, so that depth
  // 0 waits for W2 only where it scores (loads retire in issue order).
  const int n0 = ch.n;
  int32_t pq[kRPass];
#pragma unroll
  for (int k = 0; k < kRPass; ++k) pq[k] = gload(prev0 + min((tid + k * kRThreads) / NCH, n0 - 1));
  u32x4 q[kRPass];
  w1_load(q, n0, [&](int k, int) { return pq[k]; });
  __builtin_amdgcn_sched_barrier(0);
  // the wave's W2 tile, kept in registers for the whole pass
  u32x4 w[NCH];
  const int64_t tile = vc / 64;
  const int64_t tl = min(int64_t(64), int64_t(vocab) - tile * 64);
  const uint16_t* wp = w2c + tile * 64 * rank + (vc - tile * 64) * 8;
  const int64_t plane = tl * 8;
#pragma unroll
  for (int c = 0; c < NCH; ++c) w[c] = load16(wp + c * plane);
  __builtin_amdgcn_sched_barrier(0);
  // chain i's token from the thread that loaded its chunk 0 (already waited
  // for: its W1 address depends on it)
#pragma unroll
  for (int k = 0; k < kRPass; ++k) {
    const int idx = tid + k * kRThreads;
    if (idx < n0 * NCH && idx % NCH == 0) {
      s_tok[idx / NCH] = pq[k];
      s_prev[idx / NCH] = pq[k];
    }
  }
  if (tid == 0) {
    s_fail = 0;
    for (int c = 0; c < n0; ++c) {
      s_chain[c] = c;
      s_row[c] = ch.row0[c];
    }
  }
  w1_store(q, n0);

  for (int j = 0; j < ch.max_depth; ++j) {
    int n = n0;
    if (j > 0) {
      // depth j - 1's picks: every block folds the chains that go on (wave w
      // the w-th, (w + 8)-th, ... of them), block 0 also the chains that end
      // there, and block 0 writes the picks and flags
      const unsigned long long* r = rec + size_t((j - 1) & 1) * half;
      int k = 0;
      bool failed = false;
      for (int c = 0; c < ch.n; ++c) {
        const bool need = ch.depth[c] > j || (blockIdx.x == 0 && ch.depth[c] == j);
        if (!need) continue;
        if (k++ % kRWaves != wave || failed) continue;
        uint32_t tok = 0;
        bool bad = false;
        if (!fold_poll(r + size_t(c) * nblocks, nblocks, uint32_t(j), lane, wait_ticks, tok, bad)) {
          failed = true;
          if (lane == 0) s_fail = 1;
          continue;
        }
        if (lane == 0) {
          s_tok[c] = int32_t(tok);
          if (blockIdx.x == 0) {
            gstore(pick + ch.row0[c] + j - 1, int32_t(tok));
            gstore(flag + ch.row0[c] + j - 1, uint8_t(bad ? 1 : 0));
          }
        }
      }
      __syncthreads();
      if (s_fail != 0) {
        // abandoned: block 0 marks every row from depth j - 1 on with flag 2
        if (blockIdx.x == 0 && tid < ch.n)
          for (int d = j - 1; d < ch.depth[tid]; ++d) gstore(flag + ch.row0[tid] + d, uint8_t(2));
        return;
      }

      // the chains scored at this depth, in chain order
      n = 0;
      for (int c = 0; c < ch.n; ++c) n += ch.depth[c] > j ? 1 : 0;
      if (tid == 0) {
        int i = 0;
        for (int c = 0; c < ch.n; ++c)
          if (ch.depth[c] > j) {
            s_chain[i] = c;
            s_row[i] = ch.row0[c] + j;
            s_prev[i] = s_tok[c];
            ++i;
          }
      }
      __syncthreads();
      w1_load(q, n, [&](int, int i) { return s_prev[i]; });
      w1_store(q, n);
    }
    __syncthreads();

    n = __builtin_amdgcn_readfirstlane(n);  // uniform: a scalar loop count
    score_depth<NCH, kRThreads>(n, [&](int i) { return s_row[i]; }, s_prev, w, s_w1, s_key, s_bad, base,
                                stride, vc, live, vocab, tid);
    __syncthreads();
    if (tid < n) {
      uint32_t key = 0, bad = 0;
#pragma unroll
      for (int wv = 0; wv < kRWaves; ++wv) {
        key = s_key[wv][tid] > key ? s_key[wv][tid] : key;
        bad |= s_bad[wv][tid];
      }
      const unsigned long long word =
          (static_cast<unsigned long long>(j + 1) << 32) | key | (bad ? kRecBad : 0u);
      __hip_atomic_store(rec + size_t(j & 1) * half + size_t(s_chain[tid]) * nblocks + blockIdx.x, word,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // the deepest depth's picks, block 0 alone
  if (blockIdx.x != 0) return;
  const int j = ch.max_depth;
  const unsigned long long* r = rec + size_t((j - 1) & 1) * half;
  int k = 0;
  for (int c = 0; c < ch.n; ++c) {
    if (ch.depth[c] != j) continue;
    if (k++ % kRWaves != wave) continue;
    uint32_t tok = 0;
    bool bad = false;
    const bool done = fold_poll(r + size_t(c) * nblocks, nblocks, uint32_t(j), lane, wait_ticks, tok, bad);
    if (lane == 0) {
      gstore(pick + ch.row0[c] + j - 1, int32_t(done ? tok : 0u));
      gstore(flag + ch.row0[c] + j - 1, uint8_t(done ? (bad ? 1 : 0) : 2));
    }
  }
}

// Zeroes n 64-bit words (the resident form's records before a pass).
__global__ __launch_bounds__(kThreads) void markov_clear(unsigned long long* __restrict__ p, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// W2 [vocab][rank] -> tiles of 64 tokens, each [rank/8][tl][8] (tl = the
// tile's token count), one 16-byte chunk a thread.
__global__ __launch_bounds__(kThreads) void markov_pack(const uint16_t* __restrict__ w2, int64_t vocab,
                                                        int nch, uint16_t* __restrict__ w2c) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= vocab * nch) return;
  const int64_t v = t / nch;
  const int64_t c = t - v * nch;
  const int64_t tile = v / 64;
  const int64_t tl = min(int64_t(64), vocab - tile * 64);
  store16(w2c + (tile * 64 * nch + c * tl + (v - tile * 64)) * 8, load16(w2 + t * 8));
}

int64_t scan_blocks(int64_t vocab) { return (vocab + kThreads - 1) / kThreads; }

typedef void (*ScanFn)(Step, const uint16_t*, int64_t, const int32_t*, const uint16_t*, const uint16_t*, int,
                       int, const uint32_t*, uint32_t*, int32_t*, uint8_t*);

template <int... N>
constexpr auto scan_table(std::integer_sequence<int, N...>) {
  return std::array<ScanFn, sizeof...(N)>{{&markov_scan<N + 1>...}};
}
// scan_for[rank / 8 - 1]
constexpr auto scan_for = scan_table(std::make_integer_sequence<int, kMaxChunks>{});

int64_t resident_blocks(int64_t vocab) { return (vocab + kRThreads - 1) / kRThreads; }

typedef void (*ResidentFn)(Chains, const uint16_t*, int64_t, const int32_t*, const uint16_t*, const uint16_t*,
                           int, int, unsigned long long*, int32_t*, uint8_t*, uint64_t);

template <int... N>
constexpr auto resident_table(std::integer_sequence<int, N...>) {
  return std::array<ResidentFn, sizeof...(N)>{{&markov_resident<N + 1>...}};
}
// resident_for[rank / 8 - 1]
constexpr auto resident_for = resident_table(std::make_integer_sequence<int, kMaxChunks>{});

// How long a resident-form block waits for a record before it gives the
// pass up: one second of the 100 MHz clock (an exchange takes a few us).
constexpr uint64_t kWaitTicks = 100000000ull;

// How many resident-form blocks the current device holds at once for this
// rank; asked once per device and rank, kept as value + 1 so that 0 means
// not asked yet.
constexpr int kMaxDevices = 64;
std::atomic<int> g_resident_cap[kMaxDevices][kMaxChunks];

int resident_capacity(int nch) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::atomic<int>& slot = g_resident_cap[dev][nch - 1];
  int v = slot.load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, per = 0;
    int cap = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per, reinterpret_cast<const void*>(resident_for[nch - 1]), kRThreads, 0) == hipSuccess)
      cap = cus * per;
    v = cap + 1;
    slot.store(v, std::memory_order_relaxed);
  }
  return v - 1;
}

bool rank_ok(int32_t rank) { return rank >= 8 && rank <= ASV_MARKOV_MAX_RANK && rank % 8 == 0; }

}  // namespace
}  // namespace asv

extern "C" size_t asv_markov_workspace(int64_t vocab) {
  if (vocab < 1 || vocab > (int64_t(1) << 30)) return 0;
  // two halves (depths alternate), each a record per chain and block: 4 bytes
  // a 256-token block for one launch a depth, 8 a 512-token block resident
  const size_t launches = 2 * size_t(asv::scan_blocks(vocab)) * asv::kMaxChains * sizeof(uint32_t);
  const size_t resident = 2 * size_t(asv::resident_blocks(vocab)) * asv::kMaxChains * sizeof(uint64_t);
  return launches > resident ? launches : resident;
}

extern "C" int asv_markov_pack_w2(const uint16_t* w2, int64_t vocab, int32_t rank, uint16_t* w2c,
                                  void* stream) {
  if (vocab < 1 || vocab > (int64_t(1) << 30)) return ASV_E_SHAPE;
  if (!asv::rank_ok(rank)) return ASV_E_UNSUPPORTED;
  if (w2 == nullptr || w2c == nullptr || !asv::aligned16(w2) || !asv::aligned16(w2c)) return ASV_E_ARG;
  const char* a = reinterpret_cast<const char*>(w2);
  const char* b = reinterpret_cast<const char*>(w2c);
  const int64_t bytes = vocab * rank * 2;
  if (a < b + bytes && b < a + bytes) return ASV_E_ARG;
  const int64_t n = vocab * (rank / 8);
  hipLaunchKernelGGL(asv::markov_pack, dim3(unsigned((n + asv::kThreads - 1) / asv::kThreads)),
                     dim3(asv::kThreads), 0, static_cast<hipStream_t>(stream), w2, vocab, rank / 8, w2c);
  return hipGetLastError() == hipSuccess ? ASV_OK : ASV_E_HIP;
}

extern "C" int asv_markov_pick_form(const uint16_t* base, int64_t rows, int64_t row_stride,
                                    const asv_markov_chain* chains, int32_t n_chains, const int32_t* prev0,
                                    const uint16_t* w1, const uint16_t* w2c, int64_t vocab, int32_t rank,
                                    int32_t* pick, uint8_t* flag, void* workspace, size_t workspace_bytes,
                                    int32_t form, void* stream) {
  if (form != ASV_MARKOV_AUTO && form != ASV_MARKOV_LAUNCHES && form != ASV_MARKOV_RESIDENT) return ASV_E_ARG;
  if (n_chains < 0 || n_chains > ASV_MARKOV_MAX_CHAINS || rows < 0 || rows > INT_MAX)
    return ASV_E_SHAPE;
  if (vocab < 1 || vocab > (int64_t(1) << 30) || row_stride < vocab) return ASV_E_SHAPE;
  if (!asv::rank_ok(rank)) return ASV_E_UNSUPPORTED;
  if (n_chains == 0) return ASV_OK;
  if (chains == nullptr) return ASV_E_ARG;
  int max_depth = 0;
  for (int i = 0; i < n_chains; ++i) {
    const asv_markov_chain c = chains[i];
    if (c.depth < 1 || c.depth > ASV_MARKOV_MAX_DEPTH || c.row0 < 0 || int64_t(c.row0) + c.depth > rows)
      return ASV_E_SHAPE;
    for (int j = 0; j < i; ++j)
      if (c.row0 < chains[j].row0 + chains[j].depth && chains[j].row0 < c.row0 + c.depth)
        return ASV_E_SHAPE;  // two chains share a row
    max_depth = c.depth > max_depth ? c.depth : max_depth;
  }
  if (base == nullptr || prev0 == nullptr || w1 == nullptr || w2c == nullptr || pick == nullptr ||
      flag == nullptr || workspace == nullptr)
    return ASV_E_ARG;
  if ((reinterpret_cast<uintptr_t>(base) & 1u) || (reinterpret_cast<uintptr_t>(prev0) & 3u) ||
      (reinterpret_cast<uintptr_t>(pick) & 3u) || !asv::aligned16(w1) || !asv::aligned16(w2c) ||
      !asv::aligned16(workspace))
    return ASV_E_ARG;
  if (workspace_bytes < asv_markov_workspace(vocab)) return ASV_E_CAPACITY;

  hipStream_t st = static_cast<hipStream_t>(stream);

  // one resident launch when every block of it fits on the device at once
  const int64_t nres = asv::resident_blocks(vocab);
  const bool fits = nres <= asv::kRMaxBlocks && nres <= asv::resident_capacity(rank / 8);
  if (form == ASV_MARKOV_RESIDENT && !fits) return ASV_E_UNSUPPORTED;
  if (form != ASV_MARKOV_LAUNCHES && fits) {
    asv::Chains ch{};
    ch.n = n_chains;
    ch.max_depth = max_depth;
    for (int i = 0; i < n_chains; ++i) {
      ch.row0[i] = chains[i].row0;
      ch.depth[i] = chains[i].depth;
    }
    unsigned long long* rec = static_cast<unsigned long long*>(workspace);
    const int64_t words = 2 * int64_t(asv::kMaxChains) * nres;
    hipLaunchKernelGGL(asv::markov_clear, dim3(unsigned((words + asv::kThreads - 1) / asv::kThreads)),
                       dim3(asv::kThreads), 0, st, rec, words);
    if (hipGetLastError() != hipSuccess) return ASV_E_HIP;
    hipLaunchKernelGGL(asv::resident_for[rank / 8 - 1], dim3(unsigned(nres)), dim3(asv::kRThreads), 0, st, ch,
                       base, row_stride, prev0, w1, w2c, int(vocab), int(nres), rec, pick, flag, asv::kWaitTicks);
    return hipGetLastError() == hipSuccess ? ASV_OK : ASV_E_HIP;
  }

  const int nblocks = int(asv::scan_blocks(vocab));
  uint32_t* half[2] = {static_cast<uint32_t*>(workspace),
                       static_cast<uint32_t*>(workspace) + int64_t(nblocks) * asv::kMaxChains};
  asv::Step s{};
  int idx[ASV_MARKOV_MAX_CHAINS];  // chain i's index in the depth before, -1 when absent
  for (int j = 0; j < max_depth; ++j) {
    asv::Step t{};
    t.nprev = s.n;
    for (int i = 0; i < s.n; ++i) t.prow[i] = s.row[i];
    int nidx[ASV_MARKOV_MAX_CHAINS];
    for (int i = 0; i < n_chains; ++i) {
      nidx[i] = -1;
      if (chains[i].depth <= j) continue;
      t.row[t.n] = chains[i].row0 + j;
      t.src[t.n] = j == 0 ? -1 - i : idx[i];
      nidx[i] = t.n;
      ++t.n;
    }
    hipLaunchKernelGGL(asv::scan_for[rank / 8 - 1], dim3(unsigned(nblocks)), dim3(asv::kThreads), 0, st, t,
                       base, row_stride, prev0, w1, w2c, int(vocab), nblocks, half[(j + 1) & 1],
                       half[j & 1], pick, flag);
    if (hipGetLastError() != hipSuccess) return ASV_E_HIP;
    s = t;
    for (int i = 0; i < n_chains; ++i) idx[i] = nidx[i];
  }
  asv::Step f{};
  f.nprev = s.n;
  for (int i = 0; i < s.n; ++i) f.prow[i] = s.row[i];
  hipLaunchKernelGGL(asv::markov_fold, dim3(1), dim3(asv::kThreads), 0, st, f, nblocks,
                     half[(max_depth - 1) & 1], pick, flag);
  if (hipGetLastError() != hipSuccess) return ASV_E_HIP;
  return ASV_OK;
}

extern "C" int asv_markov_pick(const uint16_t* base, int64_t rows, int64_t row_stride,
                               const asv_markov_chain* chains, int32_t n_chains, const int32_t* prev0,
                               const uint16_t* w1, const uint16_t* w2c, int64_t vocab, int32_t rank,
                               int32_t* pick, uint8_t* flag, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return asv_markov_pick_form(base, rows, row_stride, chains, n_chains, prev0, w1, w2c, vocab, rank, pick,
                              flag, workspace, workspace_bytes, ASV_MARKOV_AUTO, stream);
}
