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
constexpr int kDppRowShr1 = 0x111;       // lane i <- lane i - 1 within its row (0 at the row start)
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;    // lane 15 of each row -> every lane of the next row
constexpr int kDppRowBcast31 = 0x143;    // lane 31 -> every lane of rows 2 and 3

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Lanes that the row mask leaves out, or whose source lies outside the row, read 0.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave: a shift scan inside each
// row of 16 lanes, then the row totals carried into the rows above.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_u32<kDppRowShr1>(x);
  x += dpp_u32<kDppRowShr2>(x);
  x += dpp_u32<kDppRowShr4>(x);
  x += dpp_u32<kDppRowShr8>(x);
  x += dpp_u32<kDppRowBcast15, 0xA>(x);
  x += dpp_u32<kDppRowBcast31, 0xC>(x);
  return x;
}

// Minimum (kMax false) or maximum of v over the wave, returned wave-uniform.
template <bool kMax>
__device__ __forceinline__ uint32_t wave_extreme_u32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return kMax ? max(a, b) : min(a, b); };
  v = op(v, dpp_u32<kDppRowRor8>(v));
  v = op(v, dpp_u32<kDppRowRor4>(v));
  v = op(v, dpp_u32<kDppQuadXor2>(v));
  v = op(v, dpp_u32<kDppQuadXor1>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return op(op(r0, r1), op(r2, r3));
}

// 64-bit DPP move: both halves through the same lane permutation. Lanes the
// row mask leaves out, or whose source lies outside the row, read 0.0.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = dpp_u32<kCtrl, kRowMask>((uint32_t)u);
  const uint32_t hi = dpp_u32<kCtrl, kRowMask>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the wave, returned wave-uniform: each row of 16 lanes is summed by
// DPP rotations, then the four row sums (as lane 0, 16, 32, 48 hold them) are
// added in row order. The order is fixed, so the result is reproducible.
__device__ __forceinline__ double wave_sum_f64_uniform(double v) {
  v += dpp_f64<kDppRowRor8>(v);
  v += dpp_f64<kDppRowRor4>(v);
  v += dpp_f64<kDppQuadXor2>(v);
  v += dpp_f64<kDppQuadXor1>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Maximum over the wave, returned wave-uniform.
__device__ __forceinline__ float wave_max_f32_uniform(float v) {
  v = fmaxf(v, dpp<kDppRowRor8>(v));
  v = fmaxf(v, dpp<kDppRowRor4>(v));
  v = fmaxf(v, dpp<kDppQuadXor2>(v));
  v = fmaxf(v, dpp<kDppQuadXor1>(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Inclusive prefix sum over the 64 lanes in lane order: a shift scan inside
// each row of 16, then the row totals carried into the rows above.
__device__ __forceinline__ double wave_incl_scan_f64(double x) {
  x += dpp_f64<kDppRowShr1>(x);
  x += dpp_f64<kDppRowShr2>(x);
  x += dpp_f64<kDppRowShr4>(x);
  x += dpp_f64<kDppRowShr8>(x);
  x += dpp_f64<kDppRowBcast15, 0xA>(x);
  x += dpp_f64<kDppRowBcast31, 0xC>(x);
  return x;
}

// Number of set bits of a wave-wide mask below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
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
