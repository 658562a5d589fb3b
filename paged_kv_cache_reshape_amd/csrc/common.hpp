// Shared device helpers and host-side argument checking for libpagedattn.
// gfx950 (CDNA4) only: 64-lane wavefronts, DPP row operations, permlane swaps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "pagedattn.h"

namespace pa {

// A compile-time int carried by a value (template dispatch over shapes).
template <int V>
struct IntC {
  static constexpr int value = V;
};

// ------------------------------------------------------------------ storage
// A "chunk" is the 16 bytes one lane moves with one 128-bit load or store.
struct F32 {
  using storage = float;
  static constexpr int kBytes = 4;
  static constexpr int kPerChunk = 4;  // elements per 16-byte chunk
};
struct BF16 {
  using storage = uint16_t;  // raw bfloat16 bits
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;
};

__device__ __forceinline__ uint4 load_chunk(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
// The same load for data read once per launch (the decode's K/V stream):
// marked non-temporal ("nt"), so the caches treat the lines as streaming.
// Measured on MI355X: 1-7% less time on the decode batches than plain loads
// with the same addresses; scope bits alone (sc1) changed nothing.
__device__ __forceinline__ uint4 load_stream(const void* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_chunk(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// bfloat16 -> float32 is exact: the bf16 bits are the high half of the f32.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// float32 -> bfloat16 bits, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ------------------------------------------------------------------ lanes
// DPP moves inside a 16-lane row.  Every control used here reads a lane of
// the same row that always exists, so no bound/row masking is involved.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl,
                                                    0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;           // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;           // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within each 8
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within each 16
constexpr int kDppRowRor8 = 0x128;       // lane i <- lane (i+8) mod 16

// Sum over aligned groups of kLanes lanes (kLanes in {4, 8, 16, 32}); every
// lane of a group ends with the same bits (each step adds a value and its
// partner's value, and addition is commutative).
template <int kLanes>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(kLanes == 4 || kLanes == 8 || kLanes == 16 || kLanes == 32, "");
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  if constexpr (kLanes >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (kLanes >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (kLanes >= 32) {
    // rows 0<->1 and 2<->3 exchange; both operands give row-pair sums
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x),
                                              false, false);
    x = __int_as_float(r[0]) + __int_as_float(r[1]);
  }
  return x;
}

// Maximum over aligned groups of kLanes lanes (kLanes in {4, 8, 16}).
template <int kLanes>
__device__ __forceinline__ float group_max(float x) {
  static_assert(kLanes == 4 || kLanes == 8 || kLanes == 16, "");
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  if constexpr (kLanes >= 8) x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  if constexpr (kLanes >= 16) x = fmaxf(x, dpp<kDppRowMirror>(x));
  return x;
}

// Value of the lane whose index differs in bit `kMask` (kMask in {8,16,32}).
template <int kMask>
__device__ __forceinline__ float lane_xor(float x) {
  static_assert(kMask == 8 || kMask == 16 || kMask == 32, "");
  if constexpr (kMask == 8) {
    return dpp<kDppRowRor8>(x);
  } else if constexpr (kMask == 16) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x),
                                              false, false);
    // r[0]: even rows keep own, odd rows get the even row; r[1]: the reverse.
    const bool odd_row = (__lane_id() >> 4) & 1;
    return __int_as_float(odd_row ? r[0] : r[1]);
  } else {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x),
                                              false, false);
    const bool upper = (__lane_id() >> 5) & 1;
    return __int_as_float(upper ? r[0] : r[1]);
  }
}

// ------------------------------------------------------------------ host side
void set_error(const char* fmt, ...);
void clear_error();

inline bool supported_head_dim(int d) { return d == 64 || d == 128; }
inline bool supported_block_size(int bs) { return bs == 16 || bs == 32; }
inline bool supported_dtype(int dt) { return dt == PA_DTYPE_F32 || dt == PA_DTYPE_BF16; }
inline int dtype_bytes(int dt) { return dt == PA_DTYPE_F32 ? 4 : 2; }

inline bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

constexpr int kMaxPartitionBlocks = 128;  // two table entries per lane of a wave

}  // namespace pa
