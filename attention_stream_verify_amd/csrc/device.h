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
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;

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

// Global-memory (address space 1) accesses. Pointers read out of the table
// are generic to the compiler; without the cast their loads become FLAT
// loads, which also count against the LDS wait counter, so every LDS or
// cross-lane wait would drain every load in flight.
#define ASV_GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *(const ASV_GLOBAL u32x4*)(p);
}

// Read-once streams (K/V caches): non-temporal, so they do not push other
// data out of the caches.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load((const ASV_GLOBAL u32x4*)(p));
}

__device__ __forceinline__ void store16(void* p, u32x4 v) { *(ASV_GLOBAL u32x4*)(p) = v; }

__device__ __forceinline__ void store16f(float* p, f32x4 v) { *(ASV_GLOBAL f32x4*)(p) = v; }

// Typed global load/store. Class types (table records, float2) move as raw
// words and are bit-cast, since address-space-qualified class copies are not
// expressible; every such type here is 8 bytes or a multiple of 16.
template <typename T>
__device__ __forceinline__ T gload(const T* p) {
  if constexpr (!__is_class(T)) {
    return *(const ASV_GLOBAL T*)(p);
  } else if constexpr (sizeof(T) == 8) {
    return __builtin_bit_cast(T, *(const ASV_GLOBAL unsigned long long*)(p));
  } else {
    static_assert(sizeof(T) % 16 == 0, "record size");
    struct Words {
      u32x4 w[sizeof(T) / 16];
    } v;
#pragma unroll
    for (unsigned i = 0; i < sizeof(T) / 16; ++i) v.w[i] = ((const ASV_GLOBAL u32x4*)(p))[i];
    return __builtin_bit_cast(T, v);
  }
}

// Table reads at a wave-uniform address: through the constant address space
// (the table does not change during a launch) they become scalar loads into
// SGPRs, with the scalar cache's shorter latency, instead of vector loads.
#define ASV_CONST __attribute__((address_space(4)))

template <typename T>
__device__ __forceinline__ T cload(const T* p) {
  if constexpr (!__is_class(T)) {
    return *(const ASV_CONST T*)(p);
  } else if constexpr (sizeof(T) == 8) {
    return __builtin_bit_cast(T, *(const ASV_CONST unsigned long long*)(p));
  } else {
    static_assert(sizeof(T) % 16 == 0, "record size");
    struct Words {
      u32x4 w[sizeof(T) / 16];
    } v;
#pragma unroll
    for (unsigned i = 0; i < sizeof(T) / 16; ++i) v.w[i] = ((const ASV_CONST u32x4*)(p))[i];
    return __builtin_bit_cast(T, v);
  }
}

template <typename T>
__device__ __forceinline__ void gstore(T* p, T v) {
  if constexpr (!__is_class(T)) {
    *(ASV_GLOBAL T*)(p) = v;
  } else {
    static_assert(sizeof(T) == 8, "record size");
    *(ASV_GLOBAL unsigned long long*)(p) = __builtin_bit_cast(unsigned long long, v);
  }
}

// Table records read by every lane are the same for the whole wave; moving
// their fields to scalar registers lets the compiler branch on them with
// scalar branches instead of exec masks.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ asv_tile uniform(asv_tile r) {
  return asv_tile{uni(r.stream), uni(r.row0), uni(r.nrows), uni(r.pos0)};
}
__device__ __forceinline__ asv_work uniform(asv_work r) {
  return asv_work{uni(r.tile), int8_t(uni(r.head)), int8_t(uni(r.ntiles)), int16_t(uni(r.stream)),
                  uni(r.split), uni(r.keys)};
}
__device__ __forceinline__ asv_row uniform(asv_row r) {
  return asv_row{uni(r.stream), uni(r.pos), uni(r.nkeys), uni(r.tile)};
}
__device__ __forceinline__ asv_seg uniform(asv_seg r) {
  const uint64_t p = uint64_t(r.poff);
  const int64_t poff = int64_t((uint64_t(uint32_t(uni(int(uint32_t(p >> 32))))) << 32) |
                               uint64_t(uint32_t(uni(int(uint32_t(p))))));
  return asv_seg{uni(r.row0), uni(r.rows), uni(r.keys), uni(r.cap), uni(r.split_keys),
                 uni(r.nsplit), poff, uni(r.split_tail), uni(r.nbig), {0, 0}};
}

__device__ __forceinline__ uint64_t uniform_ptr(uint64_t p) {
  return (uint64_t(uint32_t(uni(int(uint32_t(p >> 32))))) << 32) | uint64_t(uint32_t(uni(int(uint32_t(p)))));
}

// Butterflies across the 16-lane rows of a wave64 on the VALU (gfx950
// v_permlane16_swap / v_permlane32_swap): every lane gets op(x[l], x[l ^ 16])
// or op(x[l], x[l ^ 32]). No LDS traffic and no LDS wait.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ uint32_t umax_xor16(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return r[0] > r[1] ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t umax_xor32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return r[0] > r[1] ? r[0] : r[1];
}
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The table as the kernels see it: the uploaded blob plus the offsets that
// asv_seg_table_build reported.
// First key of split t of a stream (t = nsplit gives the end of the plan,
// at or past its keys).
__device__ __forceinline__ int split_start(const asv_seg& S, int t) {
  return t < S.nbig ? t * S.split_keys : S.nbig * S.split_keys + (t - S.nbig) * S.split_tail;
}

// Splits of a stream that start below key n (hold a key of [0, n)), n >= 1.
__device__ __forceinline__ int splits_before(const asv_seg& S, int n) {
  const int big = S.nbig * S.split_keys;
  if (n <= big) return (n + S.split_keys - 1) / S.split_keys;
  return S.nbig + (n - big + S.split_tail - 1) / S.split_tail;
}

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
