// Page key bounds and query-aware top-k page selection for the sparse draft.
//
// "S3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative Decoding",
// Abstract: drafting uses sparse attention to cut KV-cache reads. The pages do
// not fix the sparse rule; this library uses a query-aware page rule after the
// Quest work its reference list cites:
//   bounds:  kmin/kmax[j][d] = elementwise min/max of the keys of page j;
//   score_j = max over the GQA group's q heads of
//             scale * sum_d max(q_d * kmin_{j,d}, q_d * kmax_{j,d});
//   select:  the k = budget / P best pages by (score desc, page asc), emitted
//            in ascending page order.
// sum_d max(q kmin, q kmax) = q+ . kmax + q- . kmin with q+ = max(q, 0) and
// q- = min(q, 0), so each (page, head) score is two dot products against fixed
// vectors: for bf16 bounds, v_dot2_f32_bf16 on the packed bounds as loaded.
#include "s3r_common.h"
#include "s3r_internal.h"

namespace s3r {
namespace {

constexpr int kMaxSelectPages = 12288;  // keys staged in LDS by the top-k pass
constexpr int kSelectPagesPerBlock = 128;  // pages scored by one 256-thread block

// ---------------------------------------------------------------------------
// Bounds: one wave per (sequence, logical page, kv head). Each lane owns 8
// consecutive d of one token row; row groups cover the page's tokens and are
// folded with cross-lane min/max.
// ---------------------------------------------------------------------------
template <typename T, int kD>
__global__ __launch_bounds__(64) void bounds_kernel(BoundsArgs a) {
  constexpr int kLpr = kD / 8;      // lanes per token row
  constexpr int kRg = 64 / kLpr;    // token rows per load step
  const int lane = threadIdx.x;
  const int b = blockIdx.x / a.Hkv, h = blockIdx.x % a.Hkv;
  const int seq_len = a.seq_lens[b];
  const int n = seq_len > 0 ? (seq_len + kPage - 1) / kPage : 0;
  int first = 0;
  if (a.first_pos) first = max(a.first_pos[b], 0) / kPage;
  const int j = first + blockIdx.y;
  if (j >= n) return;
  const int valid = min(kPage, seq_len - kPage * j);
  const int phys = a.page_table[(size_t)b * a.max_pages + j];
  const int c = lane % kLpr, rg = lane / kLpr;
  const T* kbase = static_cast<const T*>(a.k_pool) + (((size_t)phys * a.Hkv + h) * kPage) * kD + 8 * c;

  float mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mn[e] = __builtin_huge_valf();
    mx[e] = -__builtin_huge_valf();
  }
  // Every row this lane covers is loaded before any is folded (one round trip).
  constexpr int kRows = kPage / kRg;
  float v[kRows][8];
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int t = rg + kRg * i;
    const T* row = kbase + (size_t)(t < valid ? t : 0) * kD;
    if constexpr (sizeof(T) == 2) {
      const uint4 raw = load_nt16<uint4>(row);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[i][2 * e] = __uint_as_float(w[e] << 16);
        v[i][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    } else {
      const f32x4 lo4 = load_nt16<f32x4>(row);
      const f32x4 hi4 = load_nt16<f32x4>(row + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[i][e] = lo4[e];
        v[i][4 + e] = hi4[e];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    if (rg + kRg * i < valid) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mn[e] = fminf(mn[e], v[i][e]);
        mx[e] = fmaxf(mx[e], v[i][e]);
      }
    }
  }
#pragma unroll
  for (int x = kLpr; x < 64; x <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mn[e] = fminf(mn[e], __shfl_xor(mn[e], x, 64));
      mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], x, 64));
    }
  }
  if (rg == 0) {
    T* out = static_cast<T*>(a.bounds) + (((size_t)phys * a.Hkv + h) * 2) * kD + 8 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (sizeof(T) == 2) {
        reinterpret_cast<uint16_t*>(out)[e] = f32_to_bf16_bits(mn[e]);
        reinterpret_cast<uint16_t*>(out)[kD + e] = f32_to_bf16_bits(mx[e]);
      } else {
        reinterpret_cast<float*>(out)[e] = mn[e];
        reinterpret_cast<float*>(out)[kD + e] = mx[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Scores: a group of D/8 lanes scores one page for every q head of the kv
// head; a wave scores 64/(D/8) pages per step.
// ---------------------------------------------------------------------------
template <typename T, int kD, int kG>
__global__ __launch_bounds__(256) void score_kernel(SelectArgs a) {
  constexpr int kLpp = kD / 8;            // lanes per page (8 d per lane)
  constexpr int kGroups = 256 / kLpp;     // page groups per block
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int seq_len = a.seq_lens[b];
  const int n = seq_len > 0 ? (seq_len + kPage - 1) / kPage : 0;
  if (a.k >= n) return;  // every page is taken; the top-k pass writes 0..n-1
  const int c = threadIdx.x % kLpp, grp = threadIdx.x / kLpp;
  const int start = blockIdx.y * kSelectPagesPerBlock;
  const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
  float* scores = a.scores + (size_t)bh * a.max_pages;
  constexpr int kIter = kSelectPagesPerBlock / kGroups;
  // All page ids first, then all bounds: one dependent round trip per block.
  int phys[kIter];
#pragma unroll
  for (int i = 0; i < kIter; ++i) {
    const int j = start + grp + kGroups * i;
    phys[i] = j < n ? pt[j] : -1;
  }

  if constexpr (sizeof(T) == 2) {
    bf16x2 qp[kG][4], qn[kG][4];
    const uint16_t* qg = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + h * kG) * kD + 8 * c;
#pragma unroll
    for (int g = 0; g < kG; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t bits = qg[(size_t)g * kD + e];
        const bool neg = (bits & 0x8000u) != 0;
        const __bf16 v = __builtin_bit_cast(__bf16, bits);
        const __bf16 z = __builtin_bit_cast(__bf16, (uint16_t)0);
        qp[g][e / 2][e % 2] = neg ? z : v;
        qn[g][e / 2][e % 2] = neg ? v : z;
      }
    const uint16_t* bb = static_cast<const uint16_t*>(a.bounds);
    uint4 kmin[kIter], kmax[kIter];
#pragma unroll
    for (int i = 0; i < kIter; ++i) {
      const uint16_t* pb = bb + ((size_t)(phys[i] < 0 ? 0 : phys[i]) * a.Hkv + h) * 2 * kD + 8 * c;
      if (phys[i] >= 0) {
        kmin[i] = load_nt16<uint4>(pb);
        kmax[i] = load_nt16<uint4>(pb + kD);
      }
    }
#pragma unroll
    for (int i = 0; i < kIter; ++i) {
      if (phys[i] < 0) continue;  // uniform within the page group
      const uint32_t mn[4] = {kmin[i].x, kmin[i].y, kmin[i].z, kmin[i].w};
      const uint32_t mx[4] = {kmax[i].x, kmax[i].y, kmax[i].z, kmax[i].w};
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
      if (c == 0) scores[start + grp + kGroups * i] = best * a.scale;
    }
  } else {
    float qp[kG][8], qn[kG][8];
    const float* qg = static_cast<const float*>(a.q) + ((size_t)b * a.Hq + h * kG) * kD + 8 * c;
#pragma unroll
    for (int g = 0; g < kG; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = qg[(size_t)g * kD + e];
        qp[g][e] = v > 0.f ? v : 0.f;
        qn[g][e] = v < 0.f ? v : 0.f;
      }
    const float* bb = static_cast<const float*>(a.bounds);
#pragma unroll
    for (int i = 0; i < kIter; ++i) {
      if (phys[i] < 0) continue;
      const float* pb = bb + ((size_t)phys[i] * a.Hkv + h) * 2 * kD + 8 * c;
      float mn[8], mx[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mn[e] = pb[e];
        mx[e] = pb[kD + e];
      }
      float best = -__builtin_huge_valf();
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc = fmaf(qp[g][e], mx[e], acc);
          acc = fmaf(qn[g][e], mn[e], acc);
        }
        best = fmaxf(best, group_sum<kLpp>(acc));
      }
      if (c == 0) scores[start + grp + kGroups * i] = best * a.scale;
    }
  }
}

// Exclusive prefix sum over the threads of a block (fixed order).
template <int kThreadsPerBlock>
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

// Float -> uint32 with the same order (larger float, larger key). -0 is folded
// into +0 first so equal scores always tie.
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Top-k: exact radix select of the k-th largest key, then a stable compaction
// in page order, which emits the kept pages ascending. Ties on the threshold
// key keep the lowest page indices. Key bits shared by every key (the common
// prefix of the block's min and max key) are skipped; the rest are resolved
// 9 bits per pass.
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;
constexpr int kDigitBits = 9;
constexpr int kBins = 1 << kDigitBits;

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(SelectArgs a) {
  extern __shared__ uint32_t keys[];
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wave_tot[kTopkThreads / 64];
  __shared__ uint32_t s_min[kTopkThreads / 64], s_max[kTopkThreads / 64];
  __shared__ uint32_t s_digit, s_krem;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int seq_len = a.seq_lens[b];
  const int n = seq_len > 0 ? (seq_len + kPage - 1) / kPage : 0;
  const int k = a.k;
  int32_t* out = a.selected + (size_t)bh * k;
  if (h == 0 && tid == 0) a.num_selected[b] = min(k, n);
  if (k >= n) {
    for (int t = tid; t < k; t += kTopkThreads) out[t] = t < n ? t : -1;
    return;
  }
  const float* sc = a.scores + (size_t)bh * a.max_pages;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  // Scores are loaded 8 per thread at a time, all in flight together.
  for (int j0 = 0; j0 < n; j0 += 8 * kTopkThreads) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + tid + kTopkThreads * e;
      v[e] = j < n ? sc[j] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + tid + kTopkThreads * e;
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
    s_min[wave] = kmin;
    s_max[wave] = kmax;
  }
  for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
  __syncthreads();
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    kmin = min(kmin, s_min[w]);
    kmax = max(kmax, s_max[w]);
  }
  const int varying = kmin == kmax ? 0 : 32 - __clz((int)(kmin ^ kmax));
  uint32_t prefix = kmin & (varying >= 32 ? 0u : ~((1u << varying) - 1u));
  uint32_t mask = varying >= 32 ? 0u : ~((1u << varying) - 1u);
  uint32_t krem = (uint32_t)k;
  for (int lo_bit = varying - kDigitBits; lo_bit > -kDigitBits; lo_bit -= kDigitBits) {
    const int shift = max(lo_bit, 0);
    const int width = lo_bit >= 0 ? kDigitBits : kDigitBits + lo_bit;
    const uint32_t dmask = (1u << width) - 1u;
    for (int j0 = 0; j0 < n; j0 += kTopkThreads) {
      const int j = j0 + tid;
      const uint32_t key = j < n ? keys[j] : 0u;
      if (j < n && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // Lane l holds the 8 bins 8l..8l+7 counted from the top digit down.
      constexpr int kPer = kBins / 64;
      uint32_t cnt[kPer], own = 0;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        cnt[e] = hist[kBins - 1 - (kPer * lane + e)];
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
          s_digit = (uint32_t)(kBins - 1 - (kPer * lane + e));
          s_krem = krem - above;
        }
        above += cnt[e];
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= dmask << shift;
    krem = s_krem;
    for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
  }
  const uint32_t thr = prefix;

  // Contiguous chunk per thread, scanned twice: equal-key ranks, then output slots.
  const int chunk = (n + kTopkThreads - 1) / kTopkThreads;
  const int lo = min(n, tid * chunk), hi = min(n, lo + chunk);
  uint32_t n_eq = 0;
  for (int j = lo; j < hi; ++j) n_eq += keys[j] == thr;
  const uint32_t eq_before = block_exclusive_scan<kTopkThreads>(n_eq, wave_tot);
  uint32_t n_take = 0, eq_rank = eq_before;
  for (int j = lo; j < hi; ++j) {
    const uint32_t key = keys[j];
    if (key > thr) ++n_take;
    else if (key == thr) n_take += (eq_rank++ < krem);
  }
  const uint32_t slot0 = block_exclusive_scan<kTopkThreads>(n_take, wave_tot);
  uint32_t slot = slot0;
  eq_rank = eq_before;
  for (int j = lo; j < hi; ++j) {
    const uint32_t key = keys[j];
    bool take = key > thr;
    if (key == thr) take = (eq_rank++ < krem);
    if (take && slot < (uint32_t)k) out[slot++] = j;
  }
}

template <typename T, int kD>
hipError_t launch_score(const SelectArgs& a, dim3 grid, hipStream_t stream) {
  switch (a.G) {
    case 1: hipLaunchKernelGGL((score_kernel<T, kD, 1>), grid, dim3(256), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((score_kernel<T, kD, 2>), grid, dim3(256), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((score_kernel<T, kD, 4>), grid, dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((score_kernel<T, kD, 8>), grid, dim3(256), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((score_kernel<T, kD, 3>), grid, dim3(256), 0, stream, a); break;
    case 5: hipLaunchKernelGGL((score_kernel<T, kD, 5>), grid, dim3(256), 0, stream, a); break;
    case 6: hipLaunchKernelGGL((score_kernel<T, kD, 6>), grid, dim3(256), 0, stream, a); break;
    case 7: hipLaunchKernelGGL((score_kernel<T, kD, 7>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int32_t select_max_pages_supported() { return kMaxSelectPages; }

size_t select_workspace_bytes(int32_t B, int32_t Hkv, int32_t max_pages) {
  return (size_t)B * Hkv * max_pages * sizeof(float);
}

hipError_t launch_bounds(const BoundsArgs& a, s3r_dtype dt, hipStream_t stream) {
  const dim3 grid((unsigned)(a.B * a.Hkv), (unsigned)a.pages_y);
  if (dt == S3R_BF16) {
    if (a.D == 128) hipLaunchKernelGGL((bounds_kernel<uint16_t, 128>), grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((bounds_kernel<uint16_t, 64>), grid, dim3(64), 0, stream, a);
  } else {
    if (a.D == 128) hipLaunchKernelGGL((bounds_kernel<float, 128>), grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((bounds_kernel<float, 64>), grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, s3r_dtype dt, hipStream_t stream) {
  const int ychunks = max(1, (a.max_pages + kSelectPagesPerBlock - 1) / kSelectPagesPerBlock);
  const dim3 grid((unsigned)(a.B * a.Hkv), (unsigned)ychunks);
  hipError_t e;
  if (dt == S3R_BF16)
    e = a.D == 128 ? launch_score<uint16_t, 128>(a, grid, stream) : launch_score<uint16_t, 64>(a, grid, stream);
  else
    e = a.D == 128 ? launch_score<float, 128>(a, grid, stream) : launch_score<float, 64>(a, grid, stream);
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)a.max_pages * sizeof(uint32_t);
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)(a.B * a.Hkv)), dim3(kTopkThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace s3r
