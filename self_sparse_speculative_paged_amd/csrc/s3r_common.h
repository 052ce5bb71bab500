// Device-side helpers shared by the libs3r kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace s3r {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kWave = 64;
constexpr int kPage = 16;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load: the data is read once, so it is fetched with the
// nontemporal hint (no reuse expected in L2 / the last-level cache).
template <typename T>
__device__ __forceinline__ T load_nt16(const void* p) {
  static_assert(sizeof(T) == 16, "16-byte loads only");
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return __builtin_bit_cast(T, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (finite inputs; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

// Butterfly over the lanes of one wave that differ in the bits of `mask_lo..`.
template <int kFirstXor, int kLastXor>
__device__ __forceinline__ float wave_xor_max(float v) {
#pragma unroll
  for (int x = kFirstXor; x <= kLastXor; x <<= 1) v = fmaxf(v, __shfl_xor(v, x, kWave));
  return v;
}

template <int kFirstXor, int kLastXor>
__device__ __forceinline__ float wave_xor_sum(float v) {
#pragma unroll
  for (int x = kFirstXor; x <= kLastXor; x <<= 1) v += __shfl_xor(v, x, kWave);
  return v;
}

// DPP lane permutations (gfx9 encodings), full-rate VALU with no LDS traffic.
constexpr int kDppRowRor8 = 0x128;       // lane i <- lane (i + 8) mod 16 within its row
constexpr int kDppRowRor4 = 0x124;       // lane i <- lane (i + 4) mod 16 within its row
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7 - i within each 8-lane half
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Sum over aligned groups of kLanes (8 or 16) lanes; every lane gets its group's sum.
template <int kLanes>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(kLanes == 8 || kLanes == 16, "group of 8 or 16 lanes");
  if constexpr (kLanes == 16) {
    v += dpp<kDppRowRor8>(v);
    v += dpp<kDppRowRor4>(v);
  } else {
    v += dpp<kDppRowHalfMirror>(v);
  }
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppQuadXor1>(v);
  return v;
}

}  // namespace s3r
