// Exact block-wide top-k of page scores, shared by the page-select kernel and
// the fused draft-step kernel.
//
// The k best pages by (score desc, page asc) are found by an exact radix
// select of the k-th largest key, then a stable compaction in page order emits
// them ascending. Ties on the threshold key keep the lowest page indices. Key
// bits shared by every key (the common prefix of the block's min and max key)
// are skipped; the rest are resolved kTopkDigitBits per pass, stopping early
// once the bin that holds the k-th key is taken whole.
//
// Keys stay in registers: thread t holds keys e * kThreads + t for e < kR, so
// a block handles n <= kR * kThreads pages (the callers check this on the host).
// Each radix pass costs one barrier: histograms rotate over three LDS buffers
// (one counting, one being cleared, one still being read) and every wave finds
// the digit itself with a DPP scan. The compaction takes one more barrier.
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

// Digit d of a radix histogram is counted at hist_slot(d). The digit scan has
// lane l read the kPer digits kTopkBins - 1 - (kPer * l + e), e < kPer, so
// lane l's digits are stored as one run of kPer slots. In a plain layout the
// lanes of one read sit kPer dwords apart, so few LDS banks serve the whole
// wave; rotating lane l's run by l / 4 spreads them over the banks.
__device__ __forceinline__ int hist_slot(uint32_t digit) {
  constexpr int kPer = kTopkBins / 64;
  const int r = kTopkBins - 1 - (int)digit;
  const int l = r / kPer;
  return l * kPer + ((r % kPer + (l >> 2)) & (kPer - 1));
}

template <int kThreads>
struct TopkShared {
  uint32_t hist[3][kTopkBins];
  uint32_t s_min[kThreads / 64], s_max[kThreads / 64];
};

// Writes the k best of scores[0..n) (requires k < n <= kR * kThreads, n < 65536)
// to out[0..k) in ascending page order. Every thread of the block calls it.
template <int kThreads, int kR>
__device__ __forceinline__ void block_topk(const float* scores, int n, int k, TopkShared<kThreads>& sh,
                           int32_t* out) {
  constexpr int kWaves = kThreads / 64;
  static_assert(kThreads % 64 == 0 && kWaves <= 16, "1 to 16 waves");
  static_assert(kR * kWaves <= kTopkBins, "per-chunk wave counts fit one histogram buffer");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Every loop over chunks skips the chunks past n with a uniform branch, so
  // the work follows n rather than the capacity kR.
  const int nchunks = (n + kThreads - 1) / kThreads;
  uint32_t key[kR];
#pragma unroll
  for (int e = 0; e < kR; ++e) {
    if (e >= nchunks) break;
    const int j = e * kThreads + tid;
    key[e] = j < n ? order_key(scores[j]) : 0u;
  }
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int e = 0; e < kR; ++e) {
    if (e >= nchunks) break;
    if (e * kThreads + tid < n) {
      kmin = min(kmin, key[e]);
      kmax = max(kmax, key[e]);
    }
  }
  kmin = wave_extreme_u32<false>(kmin);
  kmax = wave_extreme_u32<true>(kmax);
  if (lane == 0) {
    sh.s_min[wave] = kmin;
    sh.s_max[wave] = kmax;
  }
  for (int i = tid; i < kTopkBins; i += kThreads) sh.hist[0][i] = 0;
  __syncthreads();
  kmin = wave_extreme_u32<false>(lane < kWaves ? sh.s_min[lane] : 0xffffffffu);
  kmax = wave_extreme_u32<true>(lane < kWaves ? sh.s_max[lane] : 0u);

  // Invariant: the keys still in play are those with (key & mask) == prefix,
  // and krem of them belong to the top k (every key above them does).
  const int varying = kmin == kmax ? 0 : 32 - __clz((int)(kmin ^ kmax));
  uint32_t mask = varying >= 32 ? 0u : ~((1u << varying) - 1u);
  uint32_t prefix = kmin & mask;
  uint32_t krem = (uint32_t)k;
  bool whole_bin = false;
  int cur = 0;
  for (int lo_bit = varying - kTopkDigitBits; lo_bit > -kTopkDigitBits; lo_bit -= kTopkDigitBits) {
    const int shift = max(lo_bit, 0);
    const int width = lo_bit >= 0 ? kTopkDigitBits : kTopkDigitBits + lo_bit;
    const uint32_t dmask = (1u << width) - 1u;
    const int nxt = cur == 2 ? 0 : cur + 1;
    uint32_t* hist = sh.hist[cur];
    // The buffer cleared here was last read before the previous barrier.
    for (int i = tid; i < kTopkBins; i += kThreads) sh.hist[nxt][i] = 0;
#pragma unroll
    for (int e = 0; e < kR; ++e) {
      if (e >= nchunks) break;
      if (e * kThreads + tid < n && (key[e] & mask) == prefix)
        atomicAdd(&hist[hist_slot((key[e] >> shift) & dmask)], 1u);
    }
    __syncthreads();
    // Lane l holds kPer consecutive bins counted from the top digit down; the
    // one lane whose running count crosses krem names the digit.
    constexpr int kPer = kTopkBins / 64;
    uint32_t cnt[kPer], own = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      cnt[e] = hist[kPer * lane + ((e + (lane >> 2)) & (kPer - 1))];  // hist_slot of that digit
      own += cnt[e];
    }
    uint32_t above = wave_incl_scan(own) - own;
    uint32_t hit_digit = 0, hit_krem = 0, hit_count = 0;
    bool hit = false;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (above < krem && above + cnt[e] >= krem) {
        hit = true;
        hit_digit = (uint32_t)(kTopkBins - 1 - (kPer * lane + e));
        hit_krem = krem - above;
        hit_count = cnt[e];
      }
      above += cnt[e];
    }
    const uint64_t hits = __builtin_amdgcn_ballot_w64(hit);
    const int src = hits ? __builtin_ctzll(hits) : 0;
    prefix |= (uint32_t)__builtin_amdgcn_readlane(hit_digit, src) << shift;
    mask |= dmask << shift;
    krem = __builtin_amdgcn_readlane(hit_krem, src);
    const uint32_t count = __builtin_amdgcn_readlane(hit_count, src);
    cur = nxt;
    // Every key of the chosen bin is taken: the bin's low end bounds the set.
    if (count == krem) {
      whole_bin = true;
      break;
    }
  }
  // Taken: keys above thr, and the first krem keys (in page order) equal to
  // thr. A whole bin taken at once becomes thr = its low end - 1, krem = 0;
  // that low end is positive, since some key (k < n) lies below every taken one.
  const uint32_t thr = whole_bin ? prefix - 1u : prefix;
  if (whole_bin) krem = 0;

  // Compaction. Per chunk and wave, (keys equal to thr) << 16 | (keys above
  // it) goes to the buffer cleared in the last pass, which no wave reads any
  // more; an exclusive scan of those words in (chunk, wave) order, plus the
  // lanes below in the wave, gives gt(p) and eq(p), the keys above and equal
  // to thr before position p. The key at p, if taken, lands at gt(p) + min(eq(p), krem).
  uint32_t* wc = sh.hist[cur];
  // (Ballots are convergent: these two loops keep a uniform guard instead of a
  // break, which would stop them from unrolling.)
#pragma unroll
  for (int e = 0; e < kR; ++e) {
    if (e < nchunks) {
      const bool valid = e * kThreads + tid < n;
      const uint64_t bg = __builtin_amdgcn_ballot_w64(valid && key[e] > thr);
      const uint64_t be = __builtin_amdgcn_ballot_w64(valid && key[e] == thr);
      if (lane == 0) wc[e * kWaves + wave] = (uint32_t)__popcll(be) << 16 | (uint32_t)__popcll(bg);
    }
  }
  __syncthreads();
  constexpr int kChunksPerScan = 64 / kWaves;
  uint32_t carry = 0, v = 0, incl = 0;
#pragma unroll
  for (int e = 0; e < kR; ++e) {
    if (e < nchunks) {
      if (e % kChunksPerScan == 0) {
        carry += __builtin_amdgcn_readlane(incl, 63);
        const int idx = e * kWaves + lane;
        v = idx < nchunks * kWaves ? wc[idx] : 0u;
        incl = wave_incl_scan(v);
      }
      const int i = (e % kChunksPerScan) * kWaves + wave;
      const uint32_t before =
          carry + __builtin_amdgcn_readlane(incl, i) - __builtin_amdgcn_readlane(v, i);
      const int j = e * kThreads + tid;
      const bool valid = j < n;
      const bool gt = valid && key[e] > thr, eq = valid && key[e] == thr;
      const uint64_t bg = __builtin_amdgcn_ballot_w64(gt);
      const uint64_t be = __builtin_amdgcn_ballot_w64(eq);
      const uint32_t gt_before = (before & 0xffffu) + lanes_below(bg);
      const uint32_t eq_before = (before >> 16) + lanes_below(be);
      if (gt || (eq && eq_before < krem)) {
        const uint32_t slot = gt_before + min(eq_before, krem);
        if (slot < (uint32_t)k) out[slot] = j;
      }
    }
  }
}

// The selection list of one (sequence, kv head): the kk = k - nfut best of
// scores[0..n) (every page if kk >= n), ascending, then the nfut forced pages
// fut0 .. fut0 + nfut - 1 (>= n: they do not exist yet), then -1 padding.
// Forced pages below n are expected to carry +inf scores.
template <int kThreads, int kR>
__device__ __forceinline__ void select_pages(const float* scores, int n, int k, int fut0, int nfut,
                             TopkShared<kThreads>& sh, int32_t* list) {
  const int kk = k - nfut;
  if (kk > 0 && kk < n) block_topk<kThreads, kR>(scores, n, kk, sh, list);
  const int cnt = kk < n ? (kk > 0 ? kk : 0) : n;
  for (int t = threadIdx.x; t < k; t += kThreads) {
    if (t >= cnt)
      list[t] = t - cnt < nfut ? fut0 + (t - cnt) : -1;
    else if (kk >= n)
      list[t] = t;
  }
}

// Forced pages at or beyond the n existing ones: (first, count).
__device__ __forceinline__ void future_forced(int f0, int f1, int n, int& fut0, int& nfut) {
  fut0 = f0 > n ? f0 : n;
  nfut = f1 >= fut0 ? f1 - fut0 + 1 : 0;
}

}  // namespace s3r
