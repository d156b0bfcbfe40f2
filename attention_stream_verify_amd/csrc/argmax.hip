// Greedy pick and nonfinite flag of every logit row (gfx950).
//
// PR #1377 "LFM2: shared-round decode", GPU-pick commit and the kernel
// contract entry for the argmax: the pick is the first largest logit of the
// row (ties to the lower id, the host draw's rule) and a row holding a
// nonfinite logit is flagged for the host draw. NaN takes no part in the
// order; +-Inf order as usual; -0 equals +0 (float compare); a row with no
// non-NaN value picks 0.
//
// Two launches, no atomics: each block scans an 8,192-logit chunk of one row
// with 16-byte coalesced loads (4 KB per block per step; a whole chunk's
// four loads a thread are issued before its compares) and writes its
// (value, id, flag) to the workspace; a second launch folds each row's
// chunks. Many blocks per row keep small rounds (10-16 rows) from running on
// a handful of CUs. The result is exact, so the chunking never changes it.

#include <climits>
#include <mutex>

#include "device.h"

// Library-owned workspace of asv_row_argmax_noalloc: one array per GPU, in
// the code object's device memory, held until the process ends. Every chunk
// record is written by argmax_chunks before argmax_rows reads it, so nothing
// in it needs clearing between calls.
static_assert(ASV_ARGMAX_SCRATCH_BYTES % sizeof(int4) == 0, "scratch size");
static __device__ __align__(256) int4 scratch[ASV_ARGMAX_SCRATCH_BYTES / sizeof(int4)];

namespace asv {
namespace {

constexpr int kThreads = 256;
constexpr int kSteps = 4;
constexpr int kChunk = kThreads * 8 * kSteps;  // logits per block

// (v, i) beats (bv, bi): larger value, or equal value and lower id. A NaN v
// never beats anything; the start (-inf, INT_MAX) loses to any real -Inf.
__device__ __forceinline__ bool beats(float v, int i, float bv, int bi) {
  return (v > bv) || (v == bv && i < bi);
}

__device__ __forceinline__ void take(float v, int i, float& bv, int& bi) {
  if (beats(v, i, bv, bi)) {
    bv = v;
    bi = i;
  }
}

__global__ __launch_bounds__(kThreads) void argmax_chunks(const uint16_t* __restrict__ logits,
                                                          int64_t vocab, int64_t stride,
                                                          int nchunk, int4* __restrict__ ws) {
  const int row = blockIdx.x / nchunk;
  const int chunk = blockIdx.x - row * nchunk;
  const uint16_t* p = logits + int64_t(row) * stride;
  const int64_t base = int64_t(chunk) * kChunk;

  float bv = -__builtin_inff();
  int bi = INT_MAX;
  uint32_t bad = 0;
  auto scan8 = [&](const u32x4& w, int64_t e0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t x = w[k];
      bad |= ((x & 0x7F80u) == 0x7F80u) | ((x & 0x7F800000u) == 0x7F800000u);
      take(bf16_lo(x), int(e0) + 2 * k, bv, bi);
      take(bf16_hi(x), int(e0) + 2 * k + 1, bv, bi);
    }
  };
  if (base + kChunk <= vocab) {
    // a whole chunk: every load of the thread in flight before any compare
    u32x4 w[kSteps];
#pragma unroll
    for (int it = 0; it < kSteps; ++it)
      w[it] = load16(p + base + int64_t(it) * (kThreads * 8) + threadIdx.x * 8);
#pragma unroll
    for (int it = 0; it < kSteps; ++it) scan8(w[it], base + int64_t(it) * (kThreads * 8) + threadIdx.x * 8);
  } else {
#pragma unroll
  for (int it = 0; it < kSteps; ++it) {
    const int64_t e0 = base + int64_t(it) * (kThreads * 8) + threadIdx.x * 8;
    if (e0 + 8 <= vocab) {
      scan8(load16(p + e0), e0);
    } else {
      for (int j = 0; j < 8; ++j) {
        const int64_t e = e0 + j;
        if (e < vocab) {
          const uint32_t x = p[e];
          bad |= ((x & 0x7F80u) == 0x7F80u);
          take(bf16_lo(x), int(e), bv, bi);
        }
      }
    }
  }
  }

  // wave64 reduction, then across the block's 4 waves in wave order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    bad |= uint32_t(__shfl_xor(int(bad), off));
    take(ov, oi, bv, bi);
  }
  __shared__ float sv[kThreads / 64];
  __shared__ int si[kThreads / 64];
  __shared__ uint32_t sb[kThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[wave] = bv;
    si[wave] = bi;
    sb[wave] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kThreads / 64; ++w) {
      take(sv[w], si[w], bv, bi);
      bad |= sb[w];
    }
    ws[int64_t(row) * nchunk + chunk] = make_int4(__float_as_int(bv), bi, int(bad != 0), 0);
  }
}

__global__ __launch_bounds__(256) void argmax_rows(const int4* __restrict__ ws, int64_t rows,
                                                   int nchunk, int32_t* __restrict__ pick,
                                                   uint8_t* __restrict__ flag) {
  const int64_t r = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  float bv = -__builtin_inff();
  int bi = INT_MAX;
  int bad = 0;
  for (int c = 0; c < nchunk; ++c) {
    const int4 e = ws[r * nchunk + c];
    take(__int_as_float(e.x), e.y, bv, bi);
    bad |= e.z;
  }
  pick[r] = (bi == INT_MAX) ? 0 : bi;
  flag[r] = uint8_t(bad != 0);
}

int chunks_for(int64_t vocab) { return int((vocab + kChunk - 1) / kChunk); }

// Argument checks shared by both entry points; the workspace is checked by
// each caller.
int check_args(const uint16_t* logits, int64_t rows, int64_t vocab, int64_t row_stride,
               const int32_t* pick, const uint8_t* flag) {
  if (rows < 0 || vocab < 1 || vocab > (int64_t(1) << 30) || row_stride < vocab)
    return ASV_E_SHAPE;
  if (rows == 0) return ASV_OK;
  if (logits == nullptr || pick == nullptr || flag == nullptr) return ASV_E_ARG;
  if (!aligned16(logits) || row_stride % 8 != 0) return ASV_E_ARG;
  if (rows * int64_t(chunks_for(vocab)) > int64_t(INT_MAX)) return ASV_E_SHAPE;
  return ASV_OK;
}

// The two launches over a workspace of rows x chunks records.
int launch(const uint16_t* logits, int64_t rows, int64_t vocab, int64_t row_stride,
           int32_t* pick, uint8_t* flag, int4* ws, hipStream_t st) {
  const int nchunk = chunks_for(vocab);
  hipLaunchKernelGGL(argmax_chunks, dim3(unsigned(rows * nchunk)), dim3(kThreads), 0, st,
                     logits, vocab, row_stride, nchunk, ws);
  if (hipGetLastError() != hipSuccess) return ASV_E_HIP;
  hipLaunchKernelGGL(argmax_rows, dim3(unsigned((rows + 255) / 256)), dim3(256), 0, st, ws, rows,
                     nchunk, pick, flag);
  if (hipGetLastError() != hipSuccess) return ASV_E_HIP;
  return ASV_OK;
}

// The array's device address, resolved once per device with that device
// current. On the host, `scratch` names a host-side stand-in, never the
// device memory, so it is only ever used through these addresses.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(int4** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ASV_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(::scratch)) != hipSuccess || p == nullptr)
      return ASV_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<int4*>(g_scratch_ptr[dev]);
  return ASV_OK;
}

}  // namespace
}  // namespace asv

extern "C" size_t asv_row_argmax_workspace(int64_t rows, int64_t vocab) {
  if (rows <= 0 || vocab <= 0) return 0;
  return size_t(rows) * size_t(asv::chunks_for(vocab)) * sizeof(int4);
}

extern "C" int asv_row_argmax(const uint16_t* logits, int64_t rows, int64_t vocab,
                              int64_t row_stride, int32_t* pick, uint8_t* flag, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const int e = asv::check_args(logits, rows, vocab, row_stride, pick, flag);
  if (e != ASV_OK || rows == 0) return e;
  if (workspace == nullptr || !asv::aligned16(workspace)) return ASV_E_ARG;
  if (workspace_bytes < asv_row_argmax_workspace(rows, vocab)) return ASV_E_CAPACITY;
  return asv::launch(logits, rows, vocab, row_stride, pick, flag, static_cast<int4*>(workspace),
                     static_cast<hipStream_t>(stream));
}

extern "C" int asv_row_argmax_noalloc(const uint16_t* logits, int64_t rows, int64_t vocab,
                                      int64_t row_stride, int32_t* pick, uint8_t* flag,
                                      void* stream) {
  const int e = asv::check_args(logits, rows, vocab, row_stride, pick, flag);
  if (e != ASV_OK || rows == 0) return e;
  if (asv_row_argmax_workspace(rows, vocab) > size_t(ASV_ARGMAX_SCRATCH_BYTES)) return ASV_E_CAPACITY;
  int4* ws = nullptr;
  const int se = asv::scratch_for_current_device(&ws);
  if (se != ASV_OK) return se;
  return asv::launch(logits, rows, vocab, row_stride, pick, flag, ws,
                     static_cast<hipStream_t>(stream));
}
