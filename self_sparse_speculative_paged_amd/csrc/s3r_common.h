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

}  // namespace s3r
