// Page key bounds and query-aware top-k page selection for the sparse draft.
//
// "S3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative Decoding",
// Abstract: the drafter attends to a subset of the KV cache, which is what makes
// a draft step cheaper than a dense decode step. The pages do
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
#include "s3r_score.h"
#include "s3r_topk.h"

namespace s3r {
namespace {

constexpr int kMaxSelectPages = 32768;  // 32 keys per thread of the 1024-thread top-k block
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
  // Pages first .. first + span - 1 (clipped to the sequence), gridDim.y apart.
  const int j_end = (int)min((long)n, (long)first + a.span);
  for (int j = first + blockIdx.y; j < j_end; j += gridDim.y) {
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
}

// ---------------------------------------------------------------------------
// Scores: a group of D/8 lanes scores one page for every q head of the kv
// head; a wave scores 64/(D/8) pages per step.
// ---------------------------------------------------------------------------
template <typename T, int kD, int kG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kG <= 2 ? 4 : (kG <= 4 ? 3 : 2), 8)))
void score_kernel(SelectArgs a) {
  constexpr int kLpp = kD / 8;            // lanes per page (8 d per lane)
  constexpr int kGroups = 256 / kLpp;     // page groups per block
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int seq_len = a.seq_lens[b];
  const int n = seq_len > 0 ? (seq_len + kPage - 1) / kPage : 0;
  const int c = threadIdx.x % kLpp, grp = threadIdx.x / kLpp;
  const int start = blockIdx.y * kSelectPagesPerBlock;
  // Pages from `rf` on get their bounds recomputed from K first (bf16 only).
  int rf = 0x7fffffff;
  if constexpr (sizeof(T) == 2)
    if (a.refresh_from) rf = max(a.refresh_from[b], 0) / kPage;
  // A once-per-round selection always keeps its forced pages: they score +inf,
  // and those not yet in the sequence take selection slots of their own.
  const ForcedPages fp = round_forced_pages(seq_len, a.round_gamma, kPage, a.max_pages);
  int fut0, nfut;
  future_forced(fp.f0, fp.f1, n, fut0, nfut);
  auto stored = [&](int j, float s) { return j >= fp.f0 && j <= fp.f1 ? __builtin_huge_valf() : s; };
  const bool score = a.k - nfut < n;  // otherwise every page is taken: the top-k pass writes 0..n-1
  if (!score && (rf >= n || start + kSelectPagesPerBlock <= rf)) return;
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
    PageScorerBf16<kD, kG> qs;
    qs.load(static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + h * kG) * kD, c);
    const uint16_t* bb = static_cast<const uint16_t*>(a.bounds);
    // Pages before the refresh point: all bounds loads in flight together.
    uint4 kmin[kIter], kmax[kIter];
#pragma unroll
    for (int i = 0; i < kIter; ++i) {
      const int j = start + grp + kGroups * i;
      if (phys[i] >= 0 && j < rf) {
        const uint16_t* pb = bb + ((size_t)phys[i] * a.Hkv + h) * 2 * kD + 8 * c;
        kmin[i] = load_nt16<uint4>(pb);
        kmax[i] = load_nt16<uint4>(pb + kD);
      }
    }
    if (score) {
#pragma unroll
      for (int i = 0; i < kIter; ++i) {
        const int j = start + grp + kGroups * i;
        if (phys[i] < 0 || j >= rf) continue;  // uniform within the page group
        const float sc = qs.score(kmin[i], kmax[i], a.scale);
        if (c == 0) scores[j] = stored(j, sc);
      }
    }
    // Pages from the refresh point on (normally just the tail page): bounds
    // recomputed from K, written back, then scored.
    if (start + kSelectPagesPerBlock > rf) {
#pragma unroll 1
      for (int i = 0; i < kIter; ++i) {
        const int j = start + grp + kGroups * i;
        if (phys[i] < 0 || j < rf) continue;
        uint4 lo, hi;
        refresh_page_bounds_bf16<kD>(static_cast<const uint16_t*>(a.k_pool),
                                     static_cast<uint16_t*>(a.bounds_out), a.Hkv, h, phys[i],
                                     min(kPage, seq_len - kPage * j), c, lo, hi);
        if (score) {
          const float sc = qs.score(lo, hi, a.scale);
          if (c == 0) scores[j] = stored(j, sc);
        }
      }
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
      if (c == 0) scores[start + grp + kGroups * i] = stored(start + grp + kGroups * i, best * a.scale);
    }
  }
}

constexpr int kTopkThreads = 1024;

// One block per (sequence, kv head): the k best pages of its scores, ascending,
// -1 padded; every page when k >= n. A once-per-round selection appends its
// forced pages that do not exist yet (the others score +inf).
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(SelectArgs a) {
  __shared__ TopkShared<kTopkThreads> sh;
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int seq_len = a.seq_lens[b];
  const int n = seq_len > 0 ? (seq_len + kPage - 1) / kPage : 0;
  const ForcedPages fp = round_forced_pages(seq_len, a.round_gamma, kPage, a.max_pages);
  int fut0, nfut;
  future_forced(fp.f0, fp.f1, n, fut0, nfut);
  const int k = a.k;
  if (h == 0 && threadIdx.x == 0) a.num_selected[b] = min(k - nfut, n) + nfut;
  select_pages<kTopkThreads, kMaxSelectPages / kTopkThreads>(a.scores + (size_t)bh * a.max_pages, n, k,
                                                             fut0, nfut, sh, a.selected + (size_t)bh * k);
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

hipError_t launch_scores(const SelectArgs& a, s3r_dtype dt, hipStream_t stream) {
  const int ychunks = max(1, (a.max_pages + kSelectPagesPerBlock - 1) / kSelectPagesPerBlock);
  const dim3 grid((unsigned)(a.B * a.Hkv), (unsigned)ychunks);
  if (dt == S3R_BF16)
    return a.D == 128 ? launch_score<uint16_t, 128>(a, grid, stream) : launch_score<uint16_t, 64>(a, grid, stream);
  return a.D == 128 ? launch_score<float, 128>(a, grid, stream) : launch_score<float, 64>(a, grid, stream);
}

hipError_t launch_select(const SelectArgs& a, s3r_dtype dt, hipStream_t stream) {
  hipError_t e = launch_scores(a, dt, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)(a.B * a.Hkv)), dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace s3r
