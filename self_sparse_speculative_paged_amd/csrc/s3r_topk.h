// Exact block-wide top-k of page scores, shared by the page-select kernel and
// the fused draft-step kernel.
//
// The k best pages by (score desc, page asc) are found by an exact radix
// select of the k-th largest key, then a stable compaction in page order emits
// them ascending. Ties on the threshold key keep the lowest page indices. Key
// bits shared by every key (the common prefix of the block's min and max key)
// are skipped; the rest are resolved kDigitBits per pass.
#pragma once

#include "s3r_common.h"

namespace s3r {

constexpr int kTopkDigitBits = 9;
constexpr int kTopkBins = 1 << kTopkDigitBits;

// Float -> uint32 with the same order (larger float, larger key). -0 is folded
// into +0 first so equal scores always tie.
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int kThreads>
struct TopkShared {
  uint32_t hist[kTopkBins];
  uint32_t wave_tot[kThreads / 64];
  uint32_t s_min[kThreads / 64], s_max[kThreads / 64];
  uint32_t s_digit, s_krem;
};

// Exclusive prefix sum over the threads of a block (fixed order).
template <int kThreads>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  __syncthreads();
  return base + incl - v;
}

// Writes the k best of scores[0..n) (requires k < n) to out[0..k) in ascending
// page order. keys: LDS scratch of n words. Every thread of the block calls it.
template <int kThreads>
__device__ void block_topk(const float* scores, int n, int k, uint32_t* keys,
                           TopkShared<kThreads>& sh, int32_t* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  // Scores are loaded 8 per thread at a time, all in flight together.
  for (int j0 = 0; j0 < n; j0 += 8 * kThreads) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + tid + kThreads * e;
      v[e] = j < n ? scores[j] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + tid + kThreads * e;
      if (j < n) {
        const uint32_t key = order_key(v[e]);
        keys[j] = key;
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
    }
  }
  for (int x = 32; x >= 1; x >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, x, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, x, 64));
  }
  if (lane == 0) {
    sh.s_min[wave] = kmin;
    sh.s_max[wave] = kmax;
  }
  for (int i = tid; i < kTopkBins; i += kThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int w = 0; w < kThreads / 64; ++w) {
    kmin = min(kmin, sh.s_min[w]);
    kmax = max(kmax, sh.s_max[w]);
  }
  const int varying = kmin == kmax ? 0 : 32 - __clz((int)(kmin ^ kmax));
  uint32_t prefix = kmin & (varying >= 32 ? 0u : ~((1u << varying) - 1u));
  uint32_t mask = varying >= 32 ? 0u : ~((1u << varying) - 1u);
  uint32_t krem = (uint32_t)k;
  for (int lo_bit = varying - kTopkDigitBits; lo_bit > -kTopkDigitBits; lo_bit -= kTopkDigitBits) {
    const int shift = max(lo_bit, 0);
    const int width = lo_bit >= 0 ? kTopkDigitBits : kTopkDigitBits + lo_bit;
    const uint32_t dmask = (1u << width) - 1u;
    for (int j0 = 0; j0 < n; j0 += kThreads) {
      const int j = j0 + tid;
      const uint32_t key = j < n ? keys[j] : 0u;
      if (j < n && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // Lane l holds the 8 bins 8l..8l+7 counted from the top digit down.
      constexpr int kPer = kTopkBins / 64;
      uint32_t cnt[kPer], own = 0;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        cnt[e] = sh.hist[kTopkBins - 1 - (kPer * lane + e)];
        own += cnt[e];
      }
      uint32_t incl = own;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
      }
      uint32_t above = incl - own;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        if (above < krem && above + cnt[e] >= krem) {
          sh.s_digit = (uint32_t)(kTopkBins - 1 - (kPer * lane + e));
          sh.s_krem = krem - above;
        }
        above += cnt[e];
      }
    }
    __syncthreads();
    prefix |= sh.s_digit << shift;
    mask |= dmask << shift;
    krem = sh.s_krem;
    for (int i = tid; i < kTopkBins; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
  }
  const uint32_t thr = prefix;

  // Contiguous chunk per thread, scanned twice: equal-key ranks, then output slots.
  const int chunk = (n + kThreads - 1) / kThreads;
  const int lo = min(n, tid * chunk), hi = min(n, lo + chunk);
  uint32_t n_eq = 0;
  for (int j = lo; j < hi; ++j) n_eq += keys[j] == thr;
  const uint32_t eq_before = block_exclusive_scan<kThreads>(n_eq, sh.wave_tot);
  uint32_t n_take = 0, eq_rank = eq_before;
  for (int j = lo; j < hi; ++j) {
    const uint32_t key = keys[j];
    if (key > thr) ++n_take;
    else if (key == thr) n_take += (eq_rank++ < krem);
  }
  const uint32_t slot0 = block_exclusive_scan<kThreads>(n_take, sh.wave_tot);
  uint32_t slot = slot0;
  eq_rank = eq_before;
  for (int j = lo; j < hi; ++j) {
    const uint32_t key = keys[j];
    bool take = key > thr;
    if (key == thr) take = (eq_rank++ < krem);
    if (take && slot < (uint32_t)k) out[slot++] = j;
  }
}

}  // namespace s3r
