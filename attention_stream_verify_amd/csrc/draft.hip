// Draft-id gather with a failure flag (gfx950).
//
// PR #1391 "lfm2: draft with LiquidAI's DSpark drafter (--drafter)", its
// description and the held-draft fix: a device kernel moves the drafter's
// picks for every window into the id array the verify step consumes (a
// token id past the vocabulary becomes 0), and raises a per-stream flag,
// checked before the caches are committed, when a pick is invalid or came
// from a row holding a NaN or an infinity.
// The rule per entry is written out in include/asv_draft.h.
//
// One 256-thread block per stream: threads stride over the stream's span,
// and a block-wide OR of "this entry failed" becomes the stream's flag. The
// spans live in device memory the host cannot check, so every index is
// checked here against the arrays' lengths; an entry outside them fails its
// stream and is not written.

#include "device.h"
#include "asv_draft.h"

namespace asv {
namespace {

constexpr int kDraftThreads = 256;

__global__ __launch_bounds__(kDraftThreads) void draft_ids(const asv_draft_span* __restrict__ spans,
                                                           const int32_t* __restrict__ pick,
                                                           const uint8_t* __restrict__ pick_flag,
                                                           int64_t n_picks, int64_t vocab,
                                                           int32_t* __restrict__ ids, int64_t n_ids,
                                                           uint8_t* __restrict__ fail) {
  const int32_t* f = reinterpret_cast<const int32_t*>(spans + blockIdx.x);
  const asv_draft_span sp{gload(f), gload(f + 1), gload(f + 2)};
  int bad = 0;
  for (int i = threadIdx.x; i < sp.count; i += kDraftThreads) {
    const int64_t a = int64_t(sp.src) + i, b = int64_t(sp.dst) + i;
    if (a < 0 || a >= n_picks || b < 0 || b >= n_ids) {
      bad = 1;
      continue;
    }
    const int32_t p = gload(pick + a);
    const bool valid = p >= 0 && int64_t(p) < vocab;
    gstore(ids + b, valid ? p : 0);
    if (!valid || gload(pick_flag + a) != 0) bad = 1;
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) gstore(fail + blockIdx.x, uint8_t(bad ? 1 : 0));
}

}  // namespace
}  // namespace asv

extern "C" int asv_draft_ids(const asv_draft_span* spans, int32_t n_streams, const int32_t* pick,
                             const uint8_t* pick_flag, int64_t n_picks, int64_t vocab, int32_t* ids,
                             int64_t n_ids, uint8_t* fail, void* stream) {
  if (n_streams < 0 || n_picks < 0 || n_ids < 0 || vocab < 1) return ASV_E_SHAPE;
  if (n_streams == 0) return ASV_OK;
  if (spans == nullptr || fail == nullptr) return ASV_E_ARG;
  if ((n_picks > 0 && (pick == nullptr || pick_flag == nullptr)) || (n_ids > 0 && ids == nullptr))
    return ASV_E_ARG;
  if ((reinterpret_cast<uintptr_t>(spans) & 3u) || (reinterpret_cast<uintptr_t>(pick) & 3u) ||
      (reinterpret_cast<uintptr_t>(ids) & 3u))
    return ASV_E_ARG;
  hipLaunchKernelGGL(asv::draft_ids, dim3(unsigned(n_streams)), dim3(asv::kDraftThreads), 0,
                     static_cast<hipStream_t>(stream), spans, pick, pick_flag, n_picks, vocab, ids,
                     n_ids, fail);
  return hipGetLastError() == hipSuccess ? ASV_OK : ASV_E_HIP;
}
