// Device-side helpers shared by the gfx950 kernels of the shared-round
// verify step: bf16 bit conversions, 16-byte loads, the table view.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "asv.h"

namespace asv {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bit pattern, round to nearest, ties to even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// The table as the kernels see it: the uploaded blob plus the offsets that
// asv_seg_table_build reported.
struct TableView {
  const asv_seg* segs;
  const asv_row* rows;
  const asv_tile* tiles;
  const asv_work* work;
  const uint64_t* conv_state;  // [n_conv][S]
  const uint64_t* kp;          // [n_attn][S]
  const uint64_t* vp;          // [n_attn][S]
  int32_t n_streams;
  int32_t n_rows;
  int32_t n_tiles;
  int32_t n_work;
};

inline TableView make_view(const asv_table_info& in, const void* dev_blob) {
  const char* b = static_cast<const char*>(dev_blob);
  TableView v;
  v.segs = reinterpret_cast<const asv_seg*>(b + in.off_segs);
  v.rows = reinterpret_cast<const asv_row*>(b + in.off_rows);
  v.tiles = reinterpret_cast<const asv_tile*>(b + in.off_tiles);
  v.work = reinterpret_cast<const asv_work*>(b + in.off_work);
  v.conv_state = reinterpret_cast<const uint64_t*>(b + in.off_conv_state);
  v.kp = reinterpret_cast<const uint64_t*>(b + in.off_k);
  v.vp = reinterpret_cast<const uint64_t*>(b + in.off_v);
  v.n_streams = in.n_streams;
  v.n_rows = in.n_rows;
  v.n_tiles = in.n_tiles;
  v.n_work = in.n_work;
  return v;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Host-side check that an info struct came from this library's builder.
inline bool info_ok(const asv_table_info* in) {
  return in != nullptr && in->abi_version == ASV_ABI_VERSION && in->n_streams >= 1 &&
         in->n_rows >= 1 && in->n_rows <= ASV_MAX_ROWS && in->n_tiles >= 1;
}

}  // namespace asv
