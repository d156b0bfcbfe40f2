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

// A block record: bits 8..23 the order key of the block's largest score and
// bits 0..7 255 - its lane (so the lower token wins a tie inside the block),
// both 0 when every score of the block is NaN; bit 31 the nonfinite flag.
constexpr uint32_t kRecKey = 0x00FFFFFFu;
constexpr uint32_t kRecBad = 0x80000000u;

// Fold one chain's records (nblocks of them) in one wave: the largest order
// key, then the lowest token. Loads are issued by fold_load (eight a lane in
// flight) and consumed by fold_use, so a caller can put other loads after
// them.
struct FoldAcc {
  uint32_t hi, lo;  // (order key, ~token) of the best so far, (0, 0) for none
  bool bad;
};

__device__ __forceinline__ void fold_use(FoldAcc& a, const uint32_t (&e)[8], int b0, int lane) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const uint32_t key = e[u] & kRecKey;
    a.bad |= (e[u] & kRecBad) != 0u;
    if (key != 0u) {
      const uint32_t b = uint32_t(b0 + u * 64 + lane);
      const uint32_t tok = b * kThreads + (kThreads - 1 - (key & 0xFFu));
      const uint32_t hi = key >> 8, lo = ~tok;
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
    fold_use(fa, fe, 0, lane);
    for (int b0 = 64 * 8; b0 < nblocks; b0 += 64 * 8) {
      fold_load(fe, prec + int64_t(wave) * nblocks, nblocks, b0, lane);
      fold_use(fa, fe, b0, lane);
    }
    fold_done(wave, fa);
  }
  for (int ci = wave + kThreads / 64; ci < nfold; ci += kThreads / 64) {
    const uint32_t* r = prec + int64_t(ci) * nblocks;
    FoldAcc a{0u, 0u, false};
    for (int b0 = 0; b0 < nblocks; b0 += 64 * 8) {
      fold_load(fe, r, nblocks, b0, lane);
      fold_use(a, fe, b0, lane);
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

  for (int g = 0; g < st.n; g += kGroup) {
    bool ok[kGroup];
    uint32_t bv[kGroup];
    int cs[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      cs[i] = min(g + i, st.n - 1);
      const int p = s_prev[cs[i]];
      ok[i] = p >= 0 && p < vocab;
      // unconditional (a lane past the vocabulary reads the last token and
      // is not scored), so no branch makes the compiler wait for it early
      bv[i] = uint32_t(gload(base + int64_t(st.row[cs[i]]) * stride + vc));
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
      uint32_t key = (live && !nan) ? (order_key(s) << 8) | uint32_t(kThreads - 1 - tid) : 0u;
      key = wave_umax(key);
      const bool bad = __any(nonfinite) || !ok[i];
      if (lane == 0 && g + i < st.n) {
        s_key[wave][g + i] = key;
        s_bad[wave][g + i] = bad ? 1u : 0u;
      }
    }
  }
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
      fold_use(fa, e, b0, lane);
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

bool rank_ok(int32_t rank) { return rank >= 8 && rank <= ASV_MARKOV_MAX_RANK && rank % 8 == 0; }

}  // namespace
}  // namespace asv

extern "C" size_t asv_markov_workspace(int64_t vocab) {
  if (vocab < 1 || vocab > (int64_t(1) << 30)) return 0;
  // two halves (depths alternate), each a record per chain and scan block
  return 2 * size_t(asv::scan_blocks(vocab)) * asv::kMaxChains * sizeof(uint32_t);
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

extern "C" int asv_markov_pick(const uint16_t* base, int64_t rows, int64_t row_stride,
                               const asv_markov_chain* chains, int32_t n_chains, const int32_t* prev0,
                               const uint16_t* w1, const uint16_t* w2c, int64_t vocab, int32_t rank,
                               int32_t* pick, uint8_t* flag, void* workspace, size_t workspace_bytes,
                               void* stream) {
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
