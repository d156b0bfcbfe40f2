// Markov-head step of the drafter: each drafted row's pick from its logits
// plus W2 . W1[previous token] (gfx950).
//
// PR #1391 "lfm2: draft with LiquidAI's DSpark drafter (--drafter)": the
// Markov head adds W2 W1[previous token] to each block row's logits and
// takes the argmax, one row after the other (ties to the lowest token, a NaN
// score flagged); its testing notes write the score as
// bf16(base + bf16(W2 . W1[prev])), at rows x vocabulary x rank
// 1 x 128,000 x 256; the config admission caps the rank at 256. The exact
// arithmetic (float32 dot, k ascending, one rounding per term) is written
// out in include/asv_draft.h.
//
// One step is two launches, no atomics: every chain's row at depth j is
// scored by one scan launch and folded by a one-block launch, which writes
// the picks that the next step's scan reads as previous tokens.
//
// Scan: one thread per token v, 256 tokens a block. W2 is stored
// chunk-major ([rank/8][vocab][8]: the 8 coefficients k = 8c..8c+7 of token
// v at chunk c), so one 16-byte load per lane per chunk is a contiguous 1 KB
// per wave; a lane issues all rank/8 loads of its token first (up to 128
// VGPRs, 32 KB a wave in flight). The previous token and W1's row are the
// same for the whole grid, so they are read through the constant address
// space into scalar registers, and each multiply-add takes its W1 value from
// an SGPR. The dot is summed one k at a time in float32 (a fused
// multiply-add of an exact product), four chains at a time so that each
// converted W2 value serves four chains. The block's best (score, token) per
// chain and its nonfinite flag go to the workspace.

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

// The chains' rows at one depth: row[i] is chain i's logits / pick row;
// prev[i] >= 0 names the pick row holding its previous token, prev[i] < 0
// names prev0[-1 - prev[i]] (the first row's given token).
struct Step {
  int32_t n;
  int32_t row[kMaxChains];
  int32_t prev[kMaxChains];
};

// Order key of a non-NaN bf16 pattern: larger key = larger value; -0 and +0
// share a key.
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

// NCH = rank / 8, a compile-time count so that every chunk loop is straight
// code with no per-chunk guard.
template <int NCH>
__global__ __launch_bounds__(kThreads, 2) void markov_scan(Step st, const uint16_t* __restrict__ base,
                                                           int64_t stride, const int32_t* __restrict__ prev0,
                                                           const uint16_t* __restrict__ w1,
                                                           const uint16_t* __restrict__ w2c, int vocab,
                                                           const int32_t* __restrict__ pick,
                                                           int4* __restrict__ part) {
  __shared__ uint32_t s_key[kThreads / 64][kMaxChains];
  __shared__ uint32_t s_bad[kThreads / 64][kMaxChains];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int v = blockIdx.x * kThreads + tid;
  const bool live = v < vocab;
  const int vc = live ? v : vocab - 1;
  constexpr int rank = NCH * 8;

  u32x4 w[NCH];
  {
    const uint16_t* wp = w2c + int64_t(vc) * 8;
    const int64_t plane = int64_t(vocab) * 8;
#pragma unroll
    for (int c = 0; c < NCH; ++c) w[c] = load16(wp + c * plane);
  }

  for (int g = 0; g < st.n; g += kGroup) {
    // Keep W2 as raw bf16 pairs between groups (128 VGPRs); converting it
    // once for every group would hold 256 floats and spill.
#pragma unroll
    for (int c = 0; c < NCH; ++c) asm volatile("" : "+v"(w[c]));
    const uint16_t* er[kGroup];
    bool ok[kGroup];
    uint32_t bv[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const int ci = min(g + i, st.n - 1);
      const int src = st.prev[ci];
      const int p = src >= 0 ? cload(pick + src) : cload(prev0 + (-1 - src));
      ok[i] = p >= 0 && p < vocab;
      er[i] = w1 + int64_t(ok[i] ? p : 0) * rank;
      bv[i] = live ? uint32_t(gload(base + int64_t(st.row[ci]) * stride + v)) : 0u;
    }

    // W1's chunk c + 1 is requested while chunk c is summed (scalar loads,
    // one chunk ahead: 32 SGPRs a stage); the barrier keeps the scheduler
    // from pulling every chunk's scalar loads to the front.
    float acc[kGroup] = {0.f, 0.f, 0.f, 0.f};
    u32x4 e[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) e[i] = cload(reinterpret_cast<const u32x4*>(er[i]));
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      {
        u32x4 en[kGroup];
        if (c + 1 < NCH) {
          // an opaque offset: the loads can be neither merged across chunks
          // nor hoisted above this chunk
          int off = (c + 1) * 8;
          asm volatile("" : "+s"(off));
#pragma unroll
          for (int i = 0; i < kGroup; ++i) en[i] = cload(reinterpret_cast<const u32x4*>(er[i] + off));
        }
        float f[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f[2 * k] = bf16_lo(w[c][k]);
          f[2 * k + 1] = bf16_hi(w[c][k]);
        }
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            acc[i] = __builtin_fmaf(f[2 * k], bf16_lo(e[i][k]), acc[i]);
            acc[i] = __builtin_fmaf(f[2 * k + 1], bf16_hi(e[i][k]), acc[i]);
          }
        }
        if (c + 1 < NCH) {
#pragma unroll
          for (int i = 0; i < kGroup; ++i) e[i] = en[i];
        }
        __builtin_amdgcn_sched_barrier(0);
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
      if ((tid & 63) == 0 && g + i < st.n) {
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
    // (order key, token) of the block's best, or (0, 0) when every score is NaN
    const int tok = key ? blockIdx.x * kThreads + (kThreads - 1 - int(key & 0xFFu)) : 0;
    u32x4 rec;
    rec[0] = key >> 8;
    rec[1] = uint32_t(tok);
    rec[2] = bad;
    rec[3] = 0u;
    store16(part + int64_t(blockIdx.x) * kMaxChains + tid, rec);
  }
}

// One block: wave w folds chains w, w + 4, ...; lanes stride over the scan
// blocks. Larger order key wins, then the lower token.
__global__ __launch_bounds__(kThreads) void markov_fold(Step st, int nblocks, const int4* __restrict__ part,
                                                        int32_t* __restrict__ pick,
                                                        uint8_t* __restrict__ flag) {
  const int lane = threadIdx.x & 63;
  for (int ci = threadIdx.x >> 6; ci < st.n; ci += kThreads / 64) {
    uint32_t bk = 0;
    uint32_t bt = UINT_MAX;
    bool bad = false;
    // eight records in flight a lane (the loads first, then the compares)
    for (int b0 = 0; b0 < nblocks; b0 += 64 * 8) {
      int4 e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int b = b0 + u * 64 + lane;
        e[u] = b < nblocks ? gload(part + int64_t(b) * kMaxChains + ci) : make_int4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t k = uint32_t(e[u].x), t = uint32_t(e[u].y);
        if (k > bk || (k == bk && k != 0 && t < bt)) {
          bk = k;
          bt = t;
        }
        bad |= e[u].z != 0;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint32_t ok = uint32_t(__shfl_xor(int(bk), off));
      const uint32_t ot = uint32_t(__shfl_xor(int(bt), off));
      if (ok > bk || (ok == bk && ot < bt)) {
        bk = ok;
        bt = ot;
      }
    }
    bad = __any(bad);
    if (lane == 0) {
      gstore(pick + st.row[ci], int32_t(bk ? bt : 0u));
      gstore(flag + st.row[ci], uint8_t(bad ? 1 : 0));
    }
  }
}

// W2 [vocab][rank] -> chunk-major [rank/8][vocab][8], one 16-byte chunk a thread.
__global__ __launch_bounds__(kThreads) void markov_pack(const uint16_t* __restrict__ w2, int64_t vocab,
                                                        int nch, uint16_t* __restrict__ w2c) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= vocab * nch) return;
  const int64_t v = t / nch;
  const int64_t c = t - v * nch;
  store16(w2c + (c * vocab + v) * 8, load16(w2 + t * 8));
}

int64_t scan_blocks(int64_t vocab) { return (vocab + kThreads - 1) / kThreads; }

typedef void (*ScanFn)(Step, const uint16_t*, int64_t, const int32_t*, const uint16_t*, const uint16_t*, int,
                       const int32_t*, int4*);

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
  return size_t(asv::scan_blocks(vocab)) * asv::kMaxChains * sizeof(int4);
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
  int4* part = static_cast<int4*>(workspace);
  for (int j = 0; j < max_depth; ++j) {
    asv::Step s{};
    for (int i = 0; i < n_chains; ++i) {
      if (chains[i].depth <= j) continue;
      s.row[s.n] = chains[i].row0 + j;
      s.prev[s.n] = j == 0 ? -1 - i : chains[i].row0 + j - 1;
      ++s.n;
    }
    hipLaunchKernelGGL(asv::scan_for[rank / 8 - 1], dim3(unsigned(nblocks)), dim3(asv::kThreads), 0, st, s,
                       base, row_stride, prev0, w1, w2c, int(vocab), pick, part);
    if (hipGetLastError() != hipSuccess) return ASV_E_HIP;
    hipLaunchKernelGGL(asv::markov_fold, dim3(1), dim3(asv::kThreads), 0, st, s, nblocks, part, pick,
                       flag);
    if (hipGetLastError() != hipSuccess) return ASV_E_HIP;
  }
  return ASV_OK;
}
