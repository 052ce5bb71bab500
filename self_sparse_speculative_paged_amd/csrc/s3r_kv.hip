// KV commit: the KV step either side of an S3R round. New K/V rows (what a
// forward pass produced for draft or verify positions) are written into their
// pages, and the key bounds the page selection scores are brought up to date
// for the committed lengths, which also rolls back rows past them.
//
// "S3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative Decoding",
// Abstract: drafter and verifier are one model over one KV cache, so the rows
// either writes land in the pages the sparse draft ranks by their bounds.
//
// One wave per (sequence, kv head, page row): it walks the pages from the first
// written row (or the new tail, on a rollback) to the last written page or the
// tail page. Lane c of each 16-lane (D = 128) or 8-lane (D = 64) row group owns
// d = 8c .. 8c+7 of one token row. A slot's values come from the new rows when
// the call writes that slot and from the pool otherwise, so nothing written is
// read back. K rows are written as 16/32-byte runs; V is transposed inside each
// page, so each written token scatters its d values 2*P or 4*P bytes apart.
#include "s3r_common.h"
#include "s3r_internal.h"

namespace s3r {
namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = lo[e];
      v[4 + e] = hi[e];
    }
  }
}

// Stores 8 values that are exact in T (they were loaded from T).
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (__float_as_uint(v[2 * e]) >> 16) | (__float_as_uint(v[2 * e + 1]) & 0xffff0000u);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

template <typename T>
__device__ __forceinline__ void store1(T* p, float v) {
  if constexpr (sizeof(T) == 2)
    *reinterpret_cast<uint16_t*>(p) = (uint16_t)(__float_as_uint(v) >> 16);
  else
    *p = v;
}

template <typename T, int kD>
__global__ __launch_bounds__(64) void kv_commit_kernel(KvCommitArgs a) {
  constexpr int kLpr = kD / 8;    // lanes per token row
  constexpr int kRg = 64 / kLpr;  // token rows per step
  const int lane = threadIdx.x;
  const int b = blockIdx.x / a.Hkv, h = blockIdx.x % a.Hkv;
  const int c = lane % kLpr, rg = lane / kLpr;
  const int L = a.seq_lens[b];
  const int n = L > 0 ? (L + kPage - 1) / kPage : 0;
  const int first = a.first_pos[b];
  const int lo = min(first, max(L - 1, 0)) / kPage;
  int hi = max(a.count > 0 ? (first + a.count - 1) / kPage : -1, n - 1);
  hi = min(hi, a.max_pages - 1);
  const T* kn = static_cast<const T*>(a.k_new);
  const T* vn = static_cast<const T*>(a.v_new);
  T* kp = static_cast<T*>(a.k_pool);
  T* vp = static_cast<T*>(a.v_pool);
  for (int j = max(lo, 0) + blockIdx.y; j <= hi; j += gridDim.y) {
    const int phys = a.page_table[(size_t)b * a.max_pages + j];
    if (phys < 0) continue;  // an unallocated page: its rows are dropped
    const int valid = min(kPage, L - kPage * j);  // tokens of this page below L (may be <= 0)
    T* kpage = kp + ((size_t)phys * a.Hkv + h) * kPage * kD;
    T* vpage = vp + ((size_t)phys * a.Hkv + h) * kD * kPage;
    float mn[8], mx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mn[e] = __builtin_huge_valf();
      mx[e] = -__builtin_huge_valf();
    }
#pragma unroll
    for (int i = 0; i < kPage / kRg; ++i) {
      const int t = rg + kRg * i;
      const int r = kPage * j + t - first;  // row of the new block, if written
      const bool fresh = r >= 0 && r < a.count;
      float k8[8];
      if (fresh) {
        const size_t row = ((size_t)b * a.count + r) * a.Hkv + h;
        load8<T>(kn + row * kD + 8 * c, k8);
        store8<T>(kpage + (size_t)t * kD + 8 * c, k8);
        float v8[8];
        load8<T>(vn + row * kD + 8 * c, v8);
#pragma unroll
        for (int e = 0; e < 8; ++e) store1<T>(vpage + (size_t)(8 * c + e) * kPage + t, v8[e]);
      } else if (t < valid) {
        load8<T>(kpage + (size_t)t * kD + 8 * c, k8);
      }
      if (t < valid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          mn[e] = fminf(mn[e], k8[e]);
          mx[e] = fmaxf(mx[e], k8[e]);
        }
      }
    }
    if (a.bounds == nullptr || valid <= 0) continue;  // uniform over the wave
#pragma unroll
    for (int x = kLpr; x < 64; x <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mn[e] = fminf(mn[e], __shfl_xor(mn[e], x, 64));
        mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], x, 64));
      }
    }
    if (rg == 0) {
      T* out = static_cast<T*>(a.bounds) + ((size_t)phys * a.Hkv + h) * 2 * kD + 8 * c;
      store8<T>(out, mn);
      store8<T>(out + kD, mx);
    }
  }
}

}  // namespace

hipError_t launch_kv_commit(const KvCommitArgs& a, s3r_dtype dt, hipStream_t stream) {
  // Pages a call touches: those its rows land in plus a rolled-back tail; the
  // kernel strides over any more.
  int rows = (a.count + kPage - 1) / kPage + 1;
  if (rows > a.max_pages) rows = a.max_pages;
  const dim3 grid((unsigned)(a.B * a.Hkv), (unsigned)rows);
  if (dt == S3R_BF16) {
    if (a.D == 128) hipLaunchKernelGGL((kv_commit_kernel<uint16_t, 128>), grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((kv_commit_kernel<uint16_t, 64>), grid, dim3(64), 0, stream, a);
  } else {
    if (a.D == 128) hipLaunchKernelGGL((kv_commit_kernel<float, 128>), grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((kv_commit_kernel<float, 64>), grid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace s3r
