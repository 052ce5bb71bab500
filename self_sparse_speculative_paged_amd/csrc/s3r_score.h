// Query-aware page scores from bf16 key bounds, shared by the score kernel and
// the single-kernel draft step so that both rank pages bit-identically.
//
// A page group of kD/8 consecutive lanes scores one page: lane c owns
// d = 8c .. 8c+7. For each q head g of the kv head,
//   sum_d max(q_d kmin_d, q_d kmax_d) = q+ . kmax + q- . kmin,
// with q+ = max(q, 0) and q- = min(q, 0), taken as v_dot2_f32_bf16 on the
// packed bounds as loaded; the page score is scale times the maximum over g.
#pragma once

#include "s3r_common.h"
#include "s3r_internal.h"

namespace s3r {

template <int kD, int kG>
struct PageScorerBf16 {
  static constexpr int kLpp = kD / 8;  // lanes per page group
  bf16x2 qp[kG][4], qn[kG][4];

  // q0: the kv head's first q head row, [kG][kD] bf16 bits.
  __device__ __forceinline__ void load(const uint16_t* q0, int c) {
#pragma unroll
    for (int g = 0; g < kG; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t bits = q0[(size_t)g * kD + 8 * c + e];
        const bool neg = (bits & 0x8000u) != 0;
        const __bf16 v = __builtin_bit_cast(__bf16, bits);
        const __bf16 z = __builtin_bit_cast(__bf16, (uint16_t)0);
        qp[g][e / 2][e % 2] = neg ? z : v;
        qn[g][e / 2][e % 2] = neg ? v : z;
      }
  }

  // lo / hi: this lane's 8 kmin / kmax values as loaded (bf16 pairs).
  __device__ __forceinline__ float score(const uint4& lo, const uint4& hi, float scale) const {
    const uint32_t mn[4] = {lo.x, lo.y, lo.z, lo.w};
    const uint32_t mx[4] = {hi.x, hi.y, hi.z, hi.w};
    float best = -__builtin_huge_valf();
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(qp[g][p], __builtin_bit_cast(bf16x2, mx[p]), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(qn[g][p], __builtin_bit_cast(bf16x2, mn[p]), acc, false);
      }
      best = fmaxf(best, group_sum<kLpp>(acc));
    }
    return best * scale;
  }
};

// Recomputes the bf16 bounds of one page (kv head h, physical page phys,
// `valid` leading tokens) from K, writes them to bounds_out [N][Hkv][2][kD] and
// returns them packed as loaded: lane c of the page group owns d = 8c .. 8c+7.
template <int kD>
__device__ __forceinline__ void refresh_page_bounds_bf16(const uint16_t* k_pool, uint16_t* bounds_out,
                                                         int Hkv, int h, int phys, int valid, int c,
                                                         uint4& kmin, uint4& kmax) {
  const uint16_t* kb = k_pool + ((size_t)phys * Hkv + h) * kPage * kD + 8 * c;
  float mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mn[e] = __builtin_huge_valf();
    mx[e] = -__builtin_huge_valf();
  }
  // Two halves of 8 rows: each half's loads are in flight together.
#pragma unroll
  for (int t0 = 0; t0 < kPage; t0 += kPage / 2) {
    uint4 rows[kPage / 2];
#pragma unroll
    for (int t = 0; t < kPage / 2; ++t)
      rows[t] = *reinterpret_cast<const uint4*>(kb + (size_t)(t0 + t < valid ? t0 + t : 0) * kD);
#pragma unroll
    for (int t = 0; t < kPage / 2; ++t) {
      if (t0 + t < valid) {
        const uint32_t w[4] = {rows[t].x, rows[t].y, rows[t].z, rows[t].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(w[e] << 16), hi = __uint_as_float(w[e] & 0xffff0000u);
          mn[2 * e] = fminf(mn[2 * e], lo);
          mx[2 * e] = fmaxf(mx[2 * e], lo);
          mn[2 * e + 1] = fminf(mn[2 * e + 1], hi);
          mx[2 * e + 1] = fmaxf(mx[2 * e + 1], hi);
        }
      }
    }
  }
  uint32_t pmn[4], pmx[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pmn[e] = (uint32_t)f32_to_bf16_bits(mn[2 * e]) | ((uint32_t)f32_to_bf16_bits(mn[2 * e + 1]) << 16);
    pmx[e] = (uint32_t)f32_to_bf16_bits(mx[2 * e]) | ((uint32_t)f32_to_bf16_bits(mx[2 * e + 1]) << 16);
  }
  kmin = make_uint4(pmn[0], pmn[1], pmn[2], pmn[3]);
  kmax = make_uint4(pmx[0], pmx[1], pmx[2], pmx[3]);
  uint16_t* pb = bounds_out + ((size_t)phys * Hkv + h) * 2 * kD + 8 * c;
  *reinterpret_cast<uint4*>(pb) = kmin;
  *reinterpret_cast<uint4*>(pb + kD) = kmax;
}

// Where one (sequence, kv head)'s pages are scored from: its queries, pools,
// page-table row, and the refresh point rf (pages from rf on get their bounds
// recomputed from K first).
struct PageRowSource {
  const uint16_t* q0;      // the kv head's first q head row, [kG][kD] bf16 bits
  const uint16_t* k_pool;
  const uint16_t* bounds;
  uint16_t* bounds_out;
  const int32_t* pt;       // page-table row
  int Hkv, h, seq_len, rf;
  float scale;
};

// Scores pages [p0, p1) of one (sequence, kv head) into sc[j - p0] (LDS) and,
// if pt_lds is given, copies their page ids to pt_lds[j - p0]; the forced
// pages of a once-per-round selection score +inf. Pages from the refresh point
// on first get their bounds recomputed from K and written back. score == false
// (every page is taken) skips the bounds reads but still refreshes.
// A page group of kD/8 lanes scores a page; the kThreads threads take batches
// of 8 pages per group, and the next batch's page ids load while the current
// batch's bounds are in flight, so each batch costs one round trip.
template <int kD, int kG, int kThreads>
__device__ __forceinline__ void score_pages_to_lds(const PageRowSource& s, int p0, int p1, bool score,
                                                   const ForcedPages& fp, float* sc, int32_t* pt_lds) {
  constexpr int kLpp = kD / 8;
  constexpr int kGroups = kThreads / kLpp;  // pages per block-wide step
  constexpr int kIter = 8;                  // pages per page group per batch
  constexpr int kBatch = kGroups * kIter;
  const int c = threadIdx.x % kLpp, grp = threadIdx.x / kLpp;
  PageScorerBf16<kD, kG> qs;
  qs.load(s.q0, c);
  const int rf = max(s.rf, p0);
  // Refreshed pages (normally just the tail page) first, so their dependent
  // K loads overlap the first batch.
  for (int j = rf + grp; j < p1; j += kGroups) {
    const int phys = s.pt[j];
    uint4 lo, hi;
    refresh_page_bounds_bf16<kD>(s.k_pool, s.bounds_out, s.Hkv, s.h, phys, min(kPage, s.seq_len - kPage * j),
                                 c, lo, hi);
    if (score) {
      const float v = qs.score(lo, hi, s.scale);
      if (c == 0) sc[j - p0] = j >= fp.f0 && j <= fp.f1 ? __builtin_huge_valf() : v;
    }
    if (pt_lds && c == 1) pt_lds[j - p0] = phys;
  }
  const int end = min(rf, p1);
  int ids[kIter];
#pragma unroll
  for (int i = 0; i < kIter; ++i) {
    const int j = p0 + grp + kGroups * i;
    ids[i] = j < end ? s.pt[j] : -1;
  }
  for (int base = p0; base < end; base += kBatch) {
    int cur[kIter];
    uint4 lo[kIter], hi[kIter];
#pragma unroll
    for (int i = 0; i < kIter; ++i) {
      cur[i] = ids[i];
      if (score && cur[i] >= 0) {
        const uint16_t* pb = s.bounds + ((size_t)cur[i] * s.Hkv + s.h) * 2 * kD + 8 * c;
        lo[i] = load_nt16<uint4>(pb);
        hi[i] = load_nt16<uint4>(pb + kD);
      }
    }
#pragma unroll
    for (int i = 0; i < kIter; ++i) {
      const int j = base + kBatch + grp + kGroups * i;
      ids[i] = j < end ? s.pt[j] : -1;
    }
#pragma unroll
    for (int i = 0; i < kIter; ++i) {
      if (cur[i] < 0) continue;  // uniform within the page group
      const int j = base + grp + kGroups * i;
      if (score) {
        const float v = qs.score(lo[i], hi[i], s.scale);
        if (c == 0) sc[j - p0] = j >= fp.f0 && j <= fp.f1 ? __builtin_huge_valf() : v;
      }
      if (pt_lds && c == 1) pt_lds[j - p0] = cur[i];
    }
  }
}

}  // namespace s3r
