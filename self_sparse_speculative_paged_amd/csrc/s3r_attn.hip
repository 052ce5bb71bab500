// Paged GQA attention for the sparse draft and the dense verify.
//
// "S3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative Decoding",
// Abstract: drafting reads part of the KV cache and verifying reads all of it;
// as drafter and verifier are one model, both read the same cache. Both
// are softmax(scale * q K^T) V over a token set; they differ only in which
// pages are read (a selection row vs every page) and in the number of query
// positions (1 vs gamma + 1, causally masked).
//
// Each wave owns one split (a range of pages, or of selection entries) of one
// (sequence, kv head) and computes all rows = G * n_queries query rows of that
// kv head, so every K/V tile read from HBM serves the whole GQA group and all
// verify positions. The W waves of a workgroup hold splits of the same
// (sequence, kv head) and merge their partials in LDS; a combine kernel merges
// the workgroups' partials when one (sequence, kv head) spans several.
//
// bf16 path, per window of two pages (32 tokens), on MFMA 16x16x32 bf16:
//   S^T[token][row] = K[token][:] . Q[row][:]     A = K rows,  B = Q^T
//   O^T[d][row]    += V^T[d][token] P^T[token][row]  A = V^T,  B = P^T
// With the row index on the lane-within-16 axis of both products, a lane owns
// one query row in S^T, P^T and O^T alike: the softmax state is lane-local and
// a row maximum needs only two cross-lane steps. V is stored transposed inside
// each page ([D][P]) so the A operand of O^T (8 consecutive tokens of one d) is
// one 16-byte load. P is split into bf16 hi + lo parts so the P.V product keeps
// ~16 mantissa bits. The fp32 path does the same on MFMA 16x16x4 f32, one page
// per window.
//
// K/V windows reach the MFMAs through registers, loaded a few windows ahead of
// the compute. Where a dense verify's accumulators leave too few registers for
// that (head dim 128): at 33..48 rows each wave streams K through its own LDS
// ring with direct-to-LDS loads and keeps V in registers; at 49..64 rows one
// workgroup streams whole windows through a shared LDS ring, one wave per row
// block (attn_bf16_staged_kernel).
#include <climits>

#include "s3r_common.h"
#include "s3r_internal.h"
#include "s3r_score.h"
#include "s3r_topk.h"

namespace s3r {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// Pages per split of one (sequence, kv head) with n_items pages to attend: its
// pages spread evenly over all waves_per_group * n_groups splits, so a short
// sequence keeps every wave of its workgroup busy instead of leaving one long
// split to a single wave. At least 16 pages (fewer only if the plan's split is
// smaller) and at most the plan's split, which sizes the LDS window tables.
// Even, so windows of two pages never straddle splits.
__device__ __forceinline__ int split_pages(const AttnArgs& a, int n_items) {
  const int splits = a.waves_per_group * a.n_groups;
  int pps = (n_items + splits - 1) / splits;
  pps = (pps + 1) & ~1;
  const int lo = min(16, a.pages_per_split);
  return min(a.pages_per_split, max(lo, pps));
}

// Resolves the two logical pages of a window to physical pages. Invalid pages
// (past the range, -1 in a selection, or past the sequence) alias a valid page
// so every load stays in bounds; their tokens are masked.
struct WindowPages {
  int lpA, lpB;      // logical page ids, -1 when invalid
  int physA, physB;
};

template <bool kSparse>
__device__ __forceinline__ int logical_page(const int32_t* sel, int idx, int n_pages) {
  int lp = kSparse ? sel[idx] : idx;
  return (lp >= 0 && lp < n_pages) ? lp : -1;
}

// Online-softmax update of one 16-row block for one window. x[] holds this
// lane's logits (log2 units) for its row; returns p = 2^(x - m_new) in x.
template <int kTpl>
__device__ __forceinline__ float softmax_update(float (&x)[kTpl], float& m_run, float& l_run) {
  float mloc = x[0];
#pragma unroll
  for (int e = 1; e < kTpl; ++e) mloc = fmaxf(mloc, x[e]);
  mloc = wave_xor_max<16, 32>(mloc);
  const float m_new = fmaxf(m_run, mloc);
  const float msafe = (m_new == kNegInf) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m_run - msafe);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < kTpl; ++e) {
    x[e] = __builtin_amdgcn_exp2f(x[e] - msafe);
    s += x[e];
  }
  l_run = l_run * alpha + s;
  m_run = m_new;
  return alpha;
}

template <int kD, int kNB>
__device__ __forceinline__ void write_partial(const AttnArgs& a, int b, int h, int split,
                                              const float (&m_run)[kNB], float (&l_run)[kNB],
                                              const f32x4 (&acc)[kNB][kD / 16]) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  const size_t item = ((size_t)b * a.Hkv + h) * a.n_groups + split;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const float l = wave_xor_sum<16, 32>(l_run[nb]);
    const int row = 16 * nb + l16;
    if (row < a.rows) {
      if (g4 == 0) {
        a.part_ml[(item * a.rows + row) * 2 + 0] = m_run[nb];
        a.part_ml[(item * a.rows + row) * 2 + 1] = l;
      }
      float* o = a.part_o + (item * a.rows + row) * kD + 4 * g4;
#pragma unroll
      for (int mb = 0; mb < kD / 16; ++mb) *reinterpret_cast<f32x4*>(o + 16 * mb) = acc[nb][mb];
    }
  }
}

// Merges the kW per-wave partials of one workgroup (LDS regions of
// a.lds_region_bytes each, laid out o[rows][D] then ml[rows][2]) and writes the
// final rows, or one group partial when the (sequence, head) spans several
// workgroups.
template <int kD, int kW>
__device__ __forceinline__ void merge_group(const AttnArgs& a, int b, int h, int group,
                                            const char* lds) {
  const int R = a.rows;
  for (int idx = threadIdx.x; idx < R * kD; idx += 64 * kW) {
    const int row = idx / kD, d = idx % kD;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kW; ++w)
      M = fmaxf(M, reinterpret_cast<const float*>(lds + (size_t)w * a.lds_region_bytes)[R * kD + 2 * row]);
    float den = 0.f, o = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        const float* po = reinterpret_cast<const float*>(lds + (size_t)w * a.lds_region_bytes);
        const float c = __builtin_amdgcn_exp2f(po[R * kD + 2 * row] - M);
        den += c * po[R * kD + 2 * row + 1];
        o += c * po[row * kD + d];
      }
    }
    if (a.n_groups == 1) {
      const int gl = row / a.nq, i = row % a.nq;
      const size_t oi = (((size_t)b * a.nq + i) * a.Hq + h * a.G + gl) * kD + d;
      const float v = den > 0.f ? o / den : 0.f;
      if (a.out_bf16)
        static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_bits(v);
      else
        static_cast<float*>(a.out)[oi] = v;
    } else {
      const size_t item = ((size_t)b * a.Hkv + h) * a.n_groups + group;
      a.part_o[(item * R + row) * kD + d] = o;
      if (d == 0) {
        a.part_ml[(item * R + row) * 2] = M;
        a.part_ml[(item * R + row) * 2 + 1] = den;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Direct-to-LDS loads: waits placed by hand
// ---------------------------------------------------------------------------
// global_load_lds_dwordx4 writes each lane's 16 bytes at LDS address base +
// lane * 16 and counts on vmcnt like any vector load; loads return in order.
// hipcc does not order LDS reads of such a destination after the load, so every
// kernel that uses them waits on vmcnt itself before reading.
constexpr int kStagedSlot = 16384;
constexpr int kStagedLoads = 16;  // 1 KB loads per window

template <int kCount>
__device__ __forceinline__ void wait_vm() {
  static_assert(kCount >= 0 && kCount < 64, "vmcnt is 6 bits");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14;
  // expcnt and lgkmcnt left at their maxima (no wait).
  __builtin_amdgcn_s_waitcnt((kCount & 15) | (7 << 4) | (15 << 8) | ((kCount >> 4) << 14));
}

__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// This wave's loads of a window before the barrier lets it be read: the
// waves below kStagedLoads % kNB carry one load more.
template <int kNB, int kAhead>
__device__ __forceinline__ void wait_own_loads(int wave, bool full) {
  constexpr int kLo = kStagedLoads / kNB, kHi = (kStagedLoads + kNB - 1) / kNB;
  if (!full) {
    wait_vm<0>();
  } else if (wave < kStagedLoads % kNB) {
    wait_vm<kAhead * kHi>();
  } else {
    wait_vm<kAhead * kLo>();
  }
}

// LDS reads that wait for themselves (lgkmcnt(0)) in the same asm block, and
// that the compiler therefore does not order against the direct-to-LDS loads
// in flight: hipcc makes an ordinary LDS read it cannot tell apart from a
// direct-to-LDS destination wait for every such load (vmcnt(0)).
__device__ __forceinline__ uint64_t ds_read_lone(const void* p) {
  const uint32_t addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
  uint64_t r;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(addr) : "memory");
  return r;
}

__device__ __forceinline__ int4 ds_read_lone16(const void* p) {
  const uint32_t addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(addr) : "memory");
  return int4{(int)r.x, (int)r.y, (int)r.z, (int)r.w};
}

// K of one window (two pages of 16 tokens at head dim 128, 8 KB) in LDS:
// window token t at row t * 256 B, its logical 16-byte chunk c at physical
// chunk c ^ (t % 16) ^ (4 * (t / 16)), so every 16-lane group of the operand
// reads below hits all 64 banks once. Load j (0..7, 1 KB) fills rows
// 4 (j % 4) .. +3 of page j / 4; this is the lane's source offset (elements,
// within the page's kv-head block).
__device__ __forceinline__ int k_dma_offset(int j, int lane) {
  const int rr = 4 * (j & 3) + (lane >> 4);
  return rr * 128 + 8 * ((lane & 15) ^ rr ^ (4 * (j >> 2)));
}

// LDS offset of the lane's K operand for M-block mb and k-step s (the token
// order of load_bf16_k).
__device__ __forceinline__ int k_lds_offset(int mb, int s, int lane) {
  const int l16 = lane & 15, g4 = lane >> 4, pB = l16 >> 3;
  const int tok = 8 * ((l16 >> 2) & 1) + 4 * mb + (l16 & 3);
  return (16 * pB + tok) * 256 + 16 * ((4 * s + g4) ^ tok ^ (4 * pB));
}

// The eight 1 KB direct-to-LDS loads of one window's K into dst.
__device__ __forceinline__ void dma_k_window(char* dst, const uint16_t* kp, int physA, int physB,
                                             size_t page_stride, size_t head_off, const int (&goff)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint16_t* src = kp + (size_t)(j < 4 ? physA : physB) * page_stride + head_off + goff[j];
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(dst + 1024 * j), 16, 0, 0);
  }
}

// Where a wave's K ring starts in its LDS region: after its window table.
__host__ __device__ constexpr int k_ring_offset(int pages_per_split) {
  return (16 * ((pages_per_split + 1) / 2) + 255) & ~255;
}
constexpr int kKRingSlots = 3;
constexpr int kKRingBytes = kKRingSlots * 8192;

// ---------------------------------------------------------------------------
// bf16 KV
// ---------------------------------------------------------------------------
template <int kD, int kNB>
struct Bf16Tile {
  bf16x8 k[2][kD / 32];  // A operand of S^T for the two 16-token M-blocks
  bf16x8 v[kD / 16];     // A operand of O^T for each 16-wide d block
  WindowPages w;         // the window's pages
};

// K of one window: A operand of S^T for its two 16-token M-blocks.
template <int kD>
__device__ __forceinline__ void load_bf16_k(bf16x8 (&k)[2][kD / 32], const WindowPages w, const uint16_t* kp,
                                            int Hkv, int h) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  // M-block mb, row m = l16 holds window token 8*(m/4) + 4*mb + m%4: tokens
  // 0..15 come from page A (l16 < 8), 16..31 from page B.
  const int kphys = (l16 >= 8) ? w.physB : w.physA;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int slot = (8 * (l16 >> 2) + 4 * mb + (l16 & 3)) & 15;
    const uint16_t* base = kp + (((size_t)kphys * Hkv + h) * kPage + slot) * kD + 8 * g4;
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) k[mb][s] = *reinterpret_cast<const bf16x8*>(base + 32 * s);
  }
}

// V of one window: A operand of O^T for each 16-wide d block.
template <int kD>
__device__ __forceinline__ void load_bf16_v(bf16x8 (&v)[kD / 16], const WindowPages w, const uint16_t* vp,
                                            int Hkv, int h) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  // Contraction index (k-step s, lane group g4, element e) <-> d = 32 s + 8 g4 + e,
  // the same for K and Q: one K load instruction reads 64 contiguous bytes of
  // each of 16 token rows. K loads stay cached: two instructions share a line.
  // O^T A operand: lane holds V^T[d = 16*mb + l16][window tokens 8*g4 .. 8*g4+7];
  // each load instruction covers two whole 512-byte runs, streamed (nontemporal).
  const int vphys = (g4 >= 2) ? w.physB : w.physA;
  const uint16_t* vbase = vp + ((size_t)vphys * Hkv + h) * kD * kPage + l16 * kPage + 8 * (g4 & 1);
#pragma unroll
  for (int mb = 0; mb < kD / 16; ++mb) v[mb] = load_nt16<bf16x8>(vbase + (size_t)16 * mb * kPage);
}

template <int kD, int kNB>
__device__ __forceinline__ void load_bf16_tile(Bf16Tile<kD, kNB>& t, const uint16_t* kp,
                                               const uint16_t* vp, int Hkv, int h) {
  load_bf16_k<kD>(t.k, t.w, kp, Hkv, h);
  load_bf16_v<kD>(t.v, t.w, vp, Hkv, h);
}

// qsrc(nb, q) gives row block nb's query operand for every k-step; S^T is
// formed one row block at a time, so only that block's operand is live.
template <int kD, int kNB, class QSrc>
__device__ __forceinline__ void compute_bf16_kv(const bf16x8 (&k)[2][kD / 32], const bf16x8 (&v)[kD / 16],
                                                const WindowPages w, QSrc qsrc,
                                                const int (&qpos)[kNB], int min_qpos,
                                                float scale_log2, float (&m_run)[kNB],
                                                float (&l_run)[kNB], f32x4 (&acc)[kNB][kD / 16]) {
  const int lane = threadIdx.x & 63, g4 = lane >> 4;
  // Only windows reaching past the first query's position, or holding an
  // invalid page, need the mask.
  const bool need_mask = w.lpA < 0 || w.lpB < 0 || 16 * max(w.lpA, w.lpB) + 15 > min_qpos;
  f32x4 sacc[2][kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    bf16x8 q[kD / 32];
    qsrc(nb, q);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sacc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kD / 32; ++s)
        sacc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k[mb][s], q[s], sacc[mb][nb], 0, 0, 0);
    }
  }
  // This lane's tokens: window token 8*g4 + e, e = 4*mb + i.
  const int lp = (g4 >= 2) ? w.lpB : w.lpA;
  const int pos0 = 16 * lp + 8 * (g4 & 1);
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    float x[8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * mb + i] = sacc[mb][nb][i] * scale_log2;
    if (need_mask) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (lp < 0 || pos0 + e > qpos[nb]) x[e] = kNegInf;
    }
    const float alpha = softmax_update<8>(x, m_run[nb], l_run[nb]);
    if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
      for (int mb = 0; mb < kD / 16; ++mb) acc[nb][mb] *= alpha;
    }
    bf16x8 phi, plo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 hi = static_cast<__bf16>(x[e]);
      phi[e] = hi;
      plo[e] = static_cast<__bf16>(x[e] - static_cast<float>(hi));
    }
#pragma unroll
    for (int mb = 0; mb < kD / 16; ++mb) {
      acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[mb], phi, acc[nb][mb], 0, 0, 0);
      acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v[mb], plo, acc[nb][mb], 0, 0, 0);
    }
  }
}

template <int kD, int kNB>
__device__ __forceinline__ void compute_bf16_tile(const Bf16Tile<kD, kNB>& t,
                                                  const bf16x8 (&qb)[kNB][kD / 32],
                                                  const int (&qpos)[kNB], int min_qpos,
                                                  float scale_log2, float (&m_run)[kNB],
                                                  float (&l_run)[kNB], f32x4 (&acc)[kNB][kD / 16]) {
  auto qsrc = [&](int nb, bf16x8 (&q)[kD / 32]) {
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) q[s] = qb[nb][s];
  };
  compute_bf16_kv<kD, kNB>(t.k, t.v, t.w, qsrc, qpos, min_qpos, scale_log2, m_run, l_run, acc);
}

// One row block (the draft, small verify groups) fits two waves per SIMD with a
// 2-stage pipeline. Two row blocks run one wave per SIMD with three stages.
// Three row blocks keep their queries in LDS and run the K-ahead pipeline in
// the kernel instead; four keep one stage, since their accumulators and
// queries take the registers. Each depth is what fits one wave per SIMD (two
// for one row block) without spilling: at four row blocks a second stage
// spills, with the queries in LDS too (84 bytes even with V loaded at use).
template <int kNB>
constexpr int bf16_stages() { return kNB == 1 ? 2 : (kNB == 2 ? 3 : (kNB == 3 ? 2 : 1)); }
template <int kNB>
constexpr int bf16_waves_per_simd() { return kNB == 1 ? 2 : 1; }

// How a sparse workgroup gets its selection row.
constexpr int kSelGiven = 0;       // a.sel, written by s3r_page_select
constexpr int kSelFromScores = 1;  // top-k of the page scores in a.scores
constexpr int kSelScoreHere = 2;   // score every page here, then top-k

// Scores every page of (sequence b, kv head h) into sc[] (LDS) and copies its
// page ids into pt_lds[]; pages from the refresh point on first get their
// bounds recomputed from K and written back. score == false (every page is
// taken) skips the bounds reads but still refreshes and copies the ids.
template <int kD, int kG, int kThreads>
__device__ __forceinline__ void score_row_to_lds(const AttnArgs& a, int b, int h, int seq_len,
                                                 int n, bool score, const ForcedPages& fp, float* sc,
                                                 int32_t* pt_lds) {
  PageRowSource src;
  src.q0 = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + h * kG) * kD;
  src.k_pool = static_cast<const uint16_t*>(a.k_pool);
  src.bounds = static_cast<const uint16_t*>(a.bounds);
  src.bounds_out = static_cast<uint16_t*>(a.bounds_out);
  src.pt = a.page_table + (size_t)b * a.max_pages;
  src.Hkv = a.Hkv;
  src.h = h;
  src.seq_len = seq_len;
  src.rf = a.refresh_from ? min(max(a.refresh_from[b], 0) / kPage, n) : n;
  src.scale = a.sel_scale;
  score_pages_to_lds<kD, kG, kThreads>(src, 0, n, score, fp, sc, pt_lds);
}

// Each wave of a kW-wave workgroup owns one split of the same (sequence, kv
// head). Its LDS region holds first its window table, then (once its pipeline
// has drained) its (m, l, o) partial; after a barrier the workgroup merges the
// kW partials and writes either the final output (one group per (sequence,
// head)) or one group partial for the global combine.
//
// kSelect != kSelGiven (the fused draft step): the workgroup first selects its
// (sequence, kv head)'s pages itself, by an exact block top-k over the page
// scores, and attends over that list in LDS; group 0 also writes the list and
// the count out, as s3r_page_select would. With kSelScoreHere the scores come
// from this workgroup too (kG q heads per kv head, one group per (sequence,
// kv head)): LDS then holds the scores over the wave regions (dead once the
// top-k has read them), the page-table row at pt_offset and the list.
template <int kD, int kNB, bool kSparse, int kW, int kSelect = kSelGiven, int kG = 0,
          int kKeys = fused_topk_keys(kW)>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(bf16_waves_per_simd<kNB>(), 8)))
void attn_bf16_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  const int wave = kW == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = blockIdx.x % a.n_groups;
  const int slot = blockIdx.x / a.n_groups;
  const int h = slot % a.Hkv;
  const int b = a.order ? a.order[slot / a.Hkv] : slot / a.Hkv;
  const int bh = b * a.Hkv + h;
  const int seq_len = a.seq_lens[b];
  const int n_pages = seq_len > 0 ? (seq_len + kPage - 1) / kPage : 0;
  const int n_items = kSparse ? min(a.ksel, n_pages) : n_pages;
  const int pps = split_pages(a, n_items);
  const int g0 = group * kW * pps;
  // the global combine skips an empty group (group 0 still publishes the selection)
  if (g0 >= n_items && a.n_groups > 1 && !(kSelect != kSelGiven && group == 0)) return;
  const int j0 = g0 + wave * pps;
  const int j1 = min(j0 + pps, n_items);
  const bool active = j0 < n_items;

  extern __shared__ int4 lds[];
  char* region = reinterpret_cast<char*>(lds) + (size_t)wave * a.lds_region_bytes;
  const int32_t* sel_row = kSparse ? a.sel + ((size_t)b * a.Hkv + h) * a.ksel : nullptr;
  const int32_t* pt_row = a.page_table + (size_t)b * a.max_pages;
  if constexpr (kSelect != kSelGiven) {
    __shared__ TopkShared<64 * kW> sh;
    char* lds_bytes = reinterpret_cast<char*>(lds);
    int32_t* list = reinterpret_cast<int32_t*>(lds_bytes + a.list_offset);
    const int k = a.ksel;
    const float* scores = a.scores + (size_t)bh * a.max_pages;
    const ForcedPages fp = round_forced_pages(seq_len, a.round_gamma, kPage, a.max_pages);
    int fut0, nfut;
    future_forced(fp.f0, fp.f1, n_pages, fut0, nfut);
    if constexpr (kSelect == kSelScoreHere) {
      int32_t* pt_lds = reinterpret_cast<int32_t*>(lds_bytes + a.pt_offset);
      float* sc = reinterpret_cast<float*>(lds_bytes);
      score_row_to_lds<kD, kG, 64 * kW>(a, b, h, seq_len, n_pages, k - nfut < n_pages, fp, sc, pt_lds);
      __syncthreads();
      scores = sc;
      pt_row = pt_lds;
    }
    select_pages<64 * kW, kKeys>(scores, n_pages, k, fut0, nfut, sh, list);
    __syncthreads();
    if (group == 0) {
      int32_t* out = a.sel_out + (size_t)bh * k;
      for (int t = threadIdx.x; t < k; t += 64 * kW) out[t] = list[t];
      if (h == 0 && threadIdx.x == 0) a.nsel_out[b] = min(k - nfut, n_pages) + nfut;
    }
    if (g0 >= n_items && a.n_groups > 1) return;  // uniform: the whole group
    sel_row = list;
  }
  float m_run[kNB], l_run[kNB];
  f32x4 acc[kNB][kD / 16];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    m_run[nb] = kNegInf;
    l_run[nb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < kD / 16; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // This lane's query rows: B operand of S^T per row block and k-step (the
  // row on the lane-within-16 axis, d = 32 s + 8 g4 + e), and each row's position.
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  auto load_q = [&](bf16x8 (&qb)[kNB][kD / 32], int (&qpos)[kNB]) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const int row = 16 * nb + l16;
      if (row < a.rows) {
        const int gl = row / a.nq, i = row % a.nq;
        const uint16_t* qrow = qg + (((size_t)b * a.nq + i) * a.Hq + h * a.G + gl) * kD + 8 * g4;
#pragma unroll
        for (int s = 0; s < kD / 32; ++s) qb[nb][s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
        qpos[nb] = seq_len - a.nq + i;
      } else {
#pragma unroll
        for (int s = 0; s < kD / 32; ++s) qb[nb][s] = bf16x8{};
        qpos[nb] = -1;
      }
    }
  };
  // Three row blocks keep the queries in LDS (one copy per workgroup, read
  // back for each window) to free registers for a deeper K pipeline.
  // A dense verify at head dim 128 instead keeps K in an LDS ring and the
  // queries in registers (an ordinary LDS read of them would wait for every
  // direct-to-LDS load in flight).
  constexpr bool kKRing = kNB == 3 && kD == 128 && !kSparse && kSelect == kSelGiven;
  constexpr bool kQInLds = kNB == 3 && !kKRing;
  bf16x8(*q_lds)[kD / 32][64] = nullptr;
  if constexpr (kQInLds) {
    __shared__ bf16x8 q_shared[kNB][kD / 32][64];
    q_lds = q_shared;
    if (wave == 0) {
      bf16x8 qb[kNB][kD / 32];
      int qpos[kNB];
      load_q(qb, qpos);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int s = 0; s < kD / 32; ++s) q_lds[nb][s][lane] = qb[nb][s];
    }
    __syncthreads();
  }

  if (active) {
    const uint16_t* kp = static_cast<const uint16_t*>(a.k_pool);
    const uint16_t* vp = static_cast<const uint16_t*>(a.v_pool);
    const int32_t* pt = pt_row;
    const int32_t* sel = sel_row;

    bf16x8 qb[kQInLds ? 1 : kNB][kD / 32];
    int qpos[kNB];
    if constexpr (kQInLds) {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int row = 16 * nb + l16;
        qpos[nb] = row < a.rows ? seq_len - a.nq + row % a.nq : -1;
      }
    } else {
      load_q(qb, qpos);
    }
    (void)qb;

    const int min_qpos = seq_len - a.nq;
    // Resolve every window's pages once: lanes look up the split's page ids in
    // parallel (selection entry, then page table) into this wave's LDS table,
    // so the pipeline below never waits on a dependent page-table load.
    int4* win_tab = reinterpret_cast<int4*>(region);  // per window {lpA, lpB, physA, physB}
    const int n_win = (j1 - j0 + 1) / 2;
    {
      const int fallback = pt[0];
      for (int w0 = 0; w0 < n_win; w0 += 64) {
        const int wi = w0 + lane;
        if (wi < n_win) {
          const int jj = j0 + 2 * wi;
          int4 e;
          e.x = logical_page<kSparse>(sel, jj, n_pages);
          e.y = (jj + 1 < j1) ? logical_page<kSparse>(sel, jj + 1, n_pages) : -1;
          e.z = e.x >= 0 ? pt[e.x] : fallback;
          e.w = e.y >= 0 ? pt[e.y] : e.z;
          win_tab[wi] = e;
        }
      }
    }
    auto pages_of = [&](int wi) {
      const int4 e = win_tab[wi];
      WindowPages w;
      w.lpA = __builtin_amdgcn_readfirstlane(e.x);
      w.lpB = __builtin_amdgcn_readfirstlane(e.y);
      w.physA = __builtin_amdgcn_readfirstlane(e.z);
      w.physB = __builtin_amdgcn_readfirstlane(e.w);
      return w;
    };
    if constexpr (kKRing) {
      // Dense, head dim 128: K goes through this wave's own LDS ring by
      // direct-to-LDS loads and V into registers, both kAhead windows ahead of
      // the compute (32 KB in flight per wave). The wave reads only what it
      // loaded, so its own vmcnt wait orders its reads; no barrier.
      constexpr int kAhead = kKRingSlots - 1;
      char* kring = region + k_ring_offset(a.pages_per_split);
      int goff[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) goff[j] = k_dma_offset(j, lane);
      int koff[2][kD / 32];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int c = 0; c < kD / 32; ++c) koff[mb][c] = k_lds_offset(mb, c, lane);
      const size_t head_off = (size_t)h * kPage * kD;
      const size_t page_stride = (size_t)a.Hkv * kPage * kD;
      // The table is read back around loads in flight: ds_read_lone16.
      auto pages_lone = [&](int wi) {
        const int4 e = ds_read_lone16(win_tab + wi);
        WindowPages w;
        w.lpA = __builtin_amdgcn_readfirstlane(e.x);
        w.lpB = __builtin_amdgcn_readfirstlane(e.y);
        w.physA = __builtin_amdgcn_readfirstlane(e.z);
        w.physB = __builtin_amdgcn_readfirstlane(e.w);
        return w;
      };
      // Per window: V's kD/16 loads, then K's 8, in that order (a compiler
      // barrier between them), so K(i) has landed once the 16 loads of each
      // later window issued so far are all that remain in flight.
      bf16x8 vt[kKRingSlots][kD / 16];
      WindowPages wt[kKRingSlots];
      auto issue = [&](int wi, int sl) {
        wt[sl] = pages_lone(wi);
        load_bf16_v<kD>(vt[sl], wt[sl], vp, a.Hkv, h);
        asm volatile("" ::: "memory");
        dma_k_window(kring + sl * 8192, kp, wt[sl].physA, wt[sl].physB, page_stride, head_off, goff);
      };
      // Every step issues one window, the split's last one again once past
      // its end (into a slot nobody reads), so the same number of loads is in
      // flight on every path. hipcc's wait analysis merges paths by load
      // counts: with a step that issued nothing it would assume the V
      // registers still pending and wait for every load at their first use.
      wait_vm<0>();  // the table's page-table loads, before any load below is counted
#pragma unroll
      for (int j = 0; j < kAhead; ++j) issue(min(j, n_win - 1), j);
      for (int base = 0; base < n_win; base += kKRingSlots) {
#pragma unroll
        for (int s = 0; s < kKRingSlots; ++s) {
          const int i = base + s;
          if (i >= n_win) break;
          asm volatile("" ::: "memory");
          wait_lgkm0();  // the reads of the slot refilled next are done
          asm volatile("" ::: "memory");
          issue(min(i + kAhead, n_win - 1), (s + kAhead) % kKRingSlots);
          // K(i) (and V(i) before it) have landed once only the loads of the
          // kAhead windows issued since remain.
          asm volatile("" ::: "memory");
          wait_vm<16 * kAhead>();
          asm volatile("" ::: "memory");
          const char* slot = kring + s * 8192;
          bf16x8 k[2][kD / 32];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int c = 0; c < kD / 32; ++c) k[mb][c] = *reinterpret_cast<const bf16x8*>(slot + koff[mb][c]);
          auto qsrc = [&](int nb, bf16x8 (&q)[kD / 32]) {
#pragma unroll
            for (int c = 0; c < kD / 32; ++c) q[c] = qb[nb][c];
          };
          compute_bf16_kv<kD, kNB>(k, vt[s], wt[s], qsrc, qpos, min_qpos, a.scale_log2, m_run, l_run, acc);
        }
      }
      wait_vm<0>();  // the repeated tail loads land before the region takes the partial
    } else if constexpr (kQInLds) {
      // K runs kDk = 2 windows ahead of the compute and V kDv = 1: 24 KB in
      // flight per wave, in the registers a third full stage would overflow.
      // The queries come from LDS.
      constexpr int kDk = 2, kDv = 1;
      constexpr int kRk = kDk + 1, kRv = kDv + 1, kUnroll = kRk * kRv / (kRk % kRv == 0 ? kRv : 1);
      bf16x8 kt[kRk][2][kD / 32];
      bf16x8 vt[kRv][kD / 16];
      WindowPages wt[kRk];
#pragma unroll
      for (int j = 0; j < kDk; ++j) {
        if (j < n_win) {
          wt[j] = pages_of(j);
          load_bf16_k<kD>(kt[j], wt[j], kp, a.Hkv, h);
          if (j < kDv) load_bf16_v<kD>(vt[j], wt[j], vp, a.Hkv, h);
        }
      }
      for (int base = 0; base < n_win; base += kUnroll) {
#pragma unroll
        for (int s = 0; s < kUnroll; ++s) {
          const int i = base + s;
          if (i >= n_win) break;
          if (i + kDk < n_win) {
            wt[(s + kDk) % kRk] = pages_of(i + kDk);
            load_bf16_k<kD>(kt[(s + kDk) % kRk], wt[(s + kDk) % kRk], kp, a.Hkv, h);
          }
          if (i + kDv < n_win) load_bf16_v<kD>(vt[(s + kDv) % kRv], wt[(s + kDv) % kRk], vp, a.Hkv, h);
          asm volatile("" ::: "memory");  // keep the query reads in the loop
          auto qsrc = [&](int nb, bf16x8 (&q)[kD / 32]) {
#pragma unroll
            for (int c = 0; c < kD / 32; ++c) q[c] = q_lds[nb][c][lane];
          };
          compute_bf16_kv<kD, kNB>(kt[s % kRk], vt[s % kRv], wt[s % kRk], qsrc, qpos, min_qpos, a.scale_log2,
                                   m_run, l_run, acc);
        }
      }
    } else {
    // kStages-deep register pipeline: while window i is computed, the loads of
    // windows i+1 .. i+kStages-1 are in flight. Three stages fit the 512
    // registers of a single wave per SIMD up to two row blocks.
    constexpr int kStages = bf16_stages<kNB>();
    Bf16Tile<kD, kNB> t[kStages];
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) {
      if (s < n_win) {
        t[s].w = pages_of(s);
        load_bf16_tile<kD, kNB>(t[s], kp, vp, a.Hkv, h);
      }
    }
    for (int base = 0; base < n_win; base += kStages) {
#pragma unroll
      for (int s = 0; s < kStages; ++s) {
        const int i = base + s;
        if (i >= n_win) break;
        const int ip = i + kStages - 1;
        if (ip < n_win) {
          t[(s + kStages - 1) % kStages].w = pages_of(ip);
          load_bf16_tile<kD, kNB>(t[(s + kStages - 1) % kStages], kp, vp, a.Hkv, h);
        }
        compute_bf16_tile<kD, kNB>(t[s], qb, qpos, min_qpos, a.scale_log2, m_run, l_run, acc);
      }
    }
    }
  }
  // This wave's partial into its LDS region: o[rows][D], then ml[rows][2]
  // (o first keeps its 16-byte stores aligned for any row count).
  float* po = reinterpret_cast<float*>(region);
  float* pml = po + a.rows * kD;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const float l = wave_xor_sum<16, 32>(l_run[nb]);
    const int row = 16 * nb + l16;
    if (row < a.rows) {
      if (g4 == 0) {
        pml[2 * row] = m_run[nb];
        pml[2 * row + 1] = l;
      }
#pragma unroll
      for (int mb = 0; mb < kD / 16; ++mb)
        *reinterpret_cast<f32x4*>(po + row * kD + 16 * mb + 4 * g4) = acc[nb][mb];
    }
  }
  if constexpr (kW > 1) __syncthreads();
  merge_group<kD, kW>(a, b, h, group, reinterpret_cast<const char*>(lds));
}

// ---------------------------------------------------------------------------
// bf16 KV, head dim 128, four row blocks: K/V windows staged in LDS.
// ---------------------------------------------------------------------------
// At 49..64 rows one wave's accumulators and queries leave room for a single
// register stage. Here a workgroup of kNB waves streams one split of one
// (sequence, kv head) through a ring of kR LDS slots of one window each (K
// 8 KB, then V 8 KB), and wave nb computes row block nb of every window: a
// wave holds one row block's state, and the bytes in flight are set by the
// ring, not by registers. The window's sixteen 1 KB direct-to-LDS loads
// (global_load_lds_dwordx4, each lane's 16 bytes landing at lane * 16) are
// dealt round-robin over the waves. Streaming through these loads tops out
// near 5.5 TB/s on gfx950 (measured with the compute taken out), below what
// the register pipeline reaches at up to three row blocks, so only four row
// blocks take this kernel.
//
// Synchronisation, per window i, in every wave:
//   s_waitcnt vmcnt(n)  this wave's loads of window i have landed in LDS (its
//                       later loads, windows i+1 .. i+kR-2, may still fly;
//                       loads return in order);
//   s_barrier           so have every wave's; and every wave has finished
//                       reading window i-1, whose slot is refilled next;
//   issue window i+kR-1 into slot (i-1) mod kR, then read slot i mod kR.
// Each wave waits for its LDS reads (lgkmcnt(0)) before the barrier, and
// compiler barriers keep every LDS read between its two hardware barriers.
//
// LDS layout of a slot, chosen so each 16-lane group of a ds_read_b128 hits
// all 64 banks once:
//   K: window token t (0..31) at row t * 256 B; logical 16-byte chunk c of the
//      row at physical chunk c ^ (t % 16) ^ (4 * (t / 16)).
//   V: page p (A, B) at 8192 + 4096 p; d at 32 d; token half e (0: tokens
//      0..7, 1: 8..15) at physical half e ^ ((d / 8) % 2).

template <int kNB, int kR>
__global__ __launch_bounds__(64 * kNB) void attn_bf16_staged_kernel(AttnArgs a) {
  constexpr int kD = 128;
  constexpr int kLoads = (kStagedLoads + kNB - 1) / kNB;  // per wave, at most
  static_assert(kR >= 3 && (kR - 2) * kLoads < 64, "ring depth");
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = blockIdx.x % a.n_groups;
  const int pair = blockIdx.x / a.n_groups;
  const int h = pair % a.Hkv;
  const int b = a.order ? a.order[pair / a.Hkv] : pair / a.Hkv;
  const int seq_len = a.seq_lens[b];
  const int n_pages = seq_len > 0 ? (seq_len + kPage - 1) / kPage : 0;
  const int n_items = n_pages;
  const int pps = split_pages(a, n_items);
  const int j0 = group * pps;
  if (j0 >= n_items && a.n_groups > 1) return;  // the combine skips an empty group
  const int j1 = min(j0 + pps, n_items);
  const int n_win = j0 < n_items ? (j1 - j0 + 1) / 2 : 0;

  extern __shared__ int4 lds[];
  char* ring = reinterpret_cast<char*>(lds);

  // This wave's row block: the B operand of S^T per k-step and the row's position.
  const int row = 16 * wave + l16;
  bf16x8 qb[kD / 32];
  int qpos[1] = {-1};
  if (row < a.rows) {
    const int gl = row / a.nq, i = row % a.nq;
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + (((size_t)b * a.nq + i) * a.Hq + h * a.G + gl) * kD + 8 * g4;
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) qb[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
    qpos[0] = seq_len - a.nq + i;
  } else {
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) qb[s] = bf16x8{};
  }
  const int min_qpos = seq_len - a.nq;

  // Source offsets (elements, within one page's (kv head) block) of this
  // wave's loads: load j < 8 is K rows 4 (j % 4) .. +3 of page j / 4, load
  // j >= 8 is V rows d = 32 (j % 4) .. +31 of page (j - 8) / 4, each lane's
  // chunk chosen so it lands at its swizzled place.
  int goff[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int j = wave + kNB * i;
    if (j < 8) {
      goff[i] = k_dma_offset(j, lane);
    } else {
      const int d = 32 * (j & 3) + (lane >> 1);
      goff[i] = d * kPage + 8 * ((lane & 1) ^ ((d >> 3) & 1));
    }
  }
  const uint16_t* kp = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vp = static_cast<const uint16_t*>(a.v_pool);
  const size_t head_off = (size_t)h * kPage * kD;
  const size_t page_stride = (size_t)a.Hkv * kPage * kD;

  // The split's physical page pairs, one 8-byte entry per window, after the
  // ring. They are read back as each window is issued through ds_read_lone:
  // hipcc, unable to tell this table from the ring, makes an ordinary read of
  // it wait for every direct-to-LDS load in flight.
  int2* win_tab = reinterpret_cast<int2*>(ring + kR * kStagedSlot);
  {
    const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
    for (int wi = threadIdx.x; wi < n_win; wi += 64 * kNB) {
      const int lp = j0 + 2 * wi;
      win_tab[wi] = int2{pt[lp], pt[min(lp + 1, j1 - 1)]};
    }
  }
  __syncthreads();
  WindowPages wt[kR];
  auto issue = [&](int wi, int sl) {
    const uint64_t e = ds_read_lone(win_tab + wi);
    const int physA = __builtin_amdgcn_readfirstlane((int)(uint32_t)e);
    const int physB = __builtin_amdgcn_readfirstlane((int)(uint32_t)(e >> 32));
    wt[sl].lpA = j0 + 2 * wi;
    wt[sl].lpB = j0 + 2 * wi + 1 < j1 ? j0 + 2 * wi + 1 : -1;
    wt[sl].physA = wt[sl].physB = 0;
    char* dst = ring + sl * kStagedSlot;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int j = wave + kNB * i;
      if (j < kStagedLoads) {
        const int phys = (j & 4) ? physB : physA;
        const uint16_t* src = (j < 8 ? kp : vp) + (size_t)phys * page_stride + head_off + goff[i];
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)(dst + 1024 * j), 16, 0, 0);
      }
    }
  };

  // This lane's LDS read offsets within a slot (see the layout above).
  int koff[2][kD / 32];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) koff[mb][s] = k_lds_offset(mb, s, lane);
  const int voff = 8192 + 4096 * (g4 >> 1) + 32 * l16 + 16 * ((g4 & 1) ^ ((l16 >> 3) & 1));

  float m_run[1] = {kNegInf}, l_run[1] = {0.f};
  f32x4 acc[1][kD / 16];
#pragma unroll
  for (int mb = 0; mb < kD / 16; ++mb) acc[0][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto qsrc = [&](int, bf16x8 (&q)[kD / 32]) {
#pragma unroll
    for (int s = 0; s < kD / 32; ++s) q[s] = qb[s];
  };

  wait_vm<0>();  // the queries, before any load below is counted
#pragma unroll
  for (int wi = 0; wi < kR - 1; ++wi)
    if (wi < n_win) issue(wi, wi);
  for (int base = 0; base < n_win; base += kR) {
#pragma unroll
    for (int s = 0; s < kR; ++s) {
      const int wi = base + s;
      if (wi >= n_win) break;
      asm volatile("" ::: "memory");
      wait_own_loads<kNB, kR - 2>(wave, wi + kR - 2 < n_win);
      wait_lgkm0();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (wi + kR - 1 < n_win) issue(wi + kR - 1, (s + kR - 1) % kR);
      const char* slot = ring + s * kStagedSlot;
      bf16x8 k[2][kD / 32], v[kD / 16];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int c = 0; c < kD / 32; ++c) k[mb][c] = *reinterpret_cast<const bf16x8*>(slot + koff[mb][c]);
#pragma unroll
      for (int mb = 0; mb < kD / 16; ++mb) v[mb] = *reinterpret_cast<const bf16x8*>(slot + voff + 512 * mb);
      compute_bf16_kv<kD, 1>(k, v, wt[s], qsrc, qpos, min_qpos, a.scale_log2, m_run, l_run, acc);
    }
  }

  // This wave's rows: the final output, or its group's partial.
  const float l = wave_xor_sum<16, 32>(l_run[0]);
  if (row < a.rows) {
    if (a.n_groups == 1) {
      const int gl = row / a.nq, i = row % a.nq;
      const size_t ob = (((size_t)b * a.nq + i) * a.Hq + h * a.G + gl) * kD + 4 * g4;
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int mb = 0; mb < kD / 16; ++mb) {
        const f32x4 o = acc[0][mb] * inv;
        if (a.out_bf16) {
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16_bits(o[0]) | ((uint32_t)f32_to_bf16_bits(o[1]) << 16);
          pk.y = (uint32_t)f32_to_bf16_bits(o[2]) | ((uint32_t)f32_to_bf16_bits(o[3]) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + ob + 16 * mb) = pk;
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ob + 16 * mb) = o;
        }
      }
    } else {
      const size_t item = ((size_t)b * a.Hkv + h) * a.n_groups + group;
      if (g4 == 0) {
        a.part_ml[(item * a.rows + row) * 2 + 0] = m_run[0];
        a.part_ml[(item * a.rows + row) * 2 + 1] = l;
      }
      float* o = a.part_o + (item * a.rows + row) * kD + 4 * g4;
#pragma unroll
      for (int mb = 0; mb < kD / 16; ++mb) *reinterpret_cast<f32x4*>(o + 16 * mb) = acc[0][mb];
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 KV: one page (16 tokens) per window on MFMA 16x16x4 f32.
// ---------------------------------------------------------------------------
template <int kD>
struct F32Tile {
  float k[kD / 4];  // K[slot l16][d = (D/4)*g4 + s]
  f32x4 v[kD / 16]; // V^T[d = 16*mb + l16][slots 4*g4 .. 4*g4+3]
};

template <int kD>
__device__ __forceinline__ void load_f32_tile(F32Tile<kD>& t, const float* kp, const float* vp,
                                              int Hkv, int h, int phys) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  const float* kb = kp + (((size_t)phys * Hkv + h) * kPage + l16) * kD + (kD / 4) * g4;
#pragma unroll
  for (int s = 0; s < kD / 16; ++s) {
    const f32x4 v = load_nt16<f32x4>(kb + 4 * s);
#pragma unroll
    for (int e = 0; e < 4; ++e) t.k[4 * s + e] = v[e];
  }
  const float* vb = vp + ((size_t)phys * Hkv + h) * kD * kPage + l16 * kPage + 4 * g4;
#pragma unroll
  for (int mb = 0; mb < kD / 16; ++mb)
    t.v[mb] = load_nt16<f32x4>(vb + (size_t)16 * mb * kPage);
}

template <int kD, int kNB, bool kSparse>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
  const int split = blockIdx.x % a.n_groups;
  const int slot = blockIdx.x / a.n_groups;
  const int h = slot % a.Hkv;
  const int b = a.order ? a.order[slot / a.Hkv] : slot / a.Hkv;
  const int seq_len = a.seq_lens[b];
  const int n_pages = seq_len > 0 ? (seq_len + kPage - 1) / kPage : 0;
  const int n_items = kSparse ? min(a.ksel, n_pages) : n_pages;
  const int pps = split_pages(a, n_items);
  const int j0 = split * pps;
  if (j0 >= n_items) return;
  const int j1 = min(j0 + pps, n_items);

  const float* kp = static_cast<const float*>(a.k_pool);
  const float* vp = static_cast<const float*>(a.v_pool);
  const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
  const int32_t* sel = kSparse ? a.sel + ((size_t)b * a.Hkv + h) * a.ksel : nullptr;
  const float* qg = static_cast<const float*>(a.q);

  float qb[kNB][kD / 4];
  int qpos[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const int row = 16 * nb + l16;
    if (row < a.rows) {
      const int gl = row / a.nq, i = row % a.nq;
      const float* qrow = qg + (((size_t)b * a.nq + i) * a.Hq + h * a.G + gl) * kD + (kD / 4) * g4;
#pragma unroll
      for (int s = 0; s < kD / 4; ++s) qb[nb][s] = qrow[s];
      qpos[nb] = seq_len - a.nq + i;
    } else {
#pragma unroll
      for (int s = 0; s < kD / 4; ++s) qb[nb][s] = 0.f;
      qpos[nb] = -1;
    }
  }
  float m_run[kNB], l_run[kNB];
  f32x4 acc[kNB][kD / 16];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    m_run[nb] = kNegInf;
    l_run[nb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < kD / 16; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int min_qpos = seq_len - a.nq;
  const int fallback = pt[0];
  F32Tile<kD> t;
  for (int jj = j0; jj < j1; ++jj) {
    const int lp = logical_page<kSparse>(sel, jj, n_pages);
    load_f32_tile<kD>(t, kp, vp, a.Hkv, h, lp >= 0 ? pt[lp] : fallback);
    const bool need_mask = lp < 0 || 16 * lp + 15 > min_qpos;
    f32x4 sacc[kNB];
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      sacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kD / 4; ++s)
        sacc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.k[s], qb[nb][s], sacc[nb], 0, 0, 0);
    }
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = sacc[nb][i] * a.scale_log2;
        if (need_mask && (lp < 0 || 16 * lp + 4 * g4 + i > qpos[nb])) x[i] = kNegInf;
      }
      const float alpha = softmax_update<4>(x, m_run[nb], l_run[nb]);
      if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
        for (int mb = 0; mb < kD / 16; ++mb) acc[nb][mb] *= alpha;
      }
#pragma unroll
      for (int mb = 0; mb < kD / 16; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.v[mb][i], x[i], acc[nb][mb], 0, 0, 0);
    }
  }
  write_partial<kD, kNB>(a, b, h, split, m_run, l_run, acc);
}

// ---------------------------------------------------------------------------
// Longest-first order: order[r] = the sequence of rank r by (length desc, index
// asc). Thread b counts the sequences ranked before it over the lengths staged
// in LDS, 1024 at a time, four per LDS read; slots past B hold INT_MIN, which
// never ranks before a sequence (its index is past every b).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void order_by_length_kernel(const int32_t* seq_lens, int B,
                                                              int32_t* order) {
  __shared__ int4 lens4[256];
  int32_t* lens = reinterpret_cast<int32_t*>(lens4);
  const int b = blockIdx.x * 256 + threadIdx.x;
  const int L = b < B ? seq_lens[b] : 0;
  int rank = 0;
  for (int c0 = 0; c0 < B; c0 += 1024) {
    __syncthreads();
    for (int c = threadIdx.x; c < 1024; c += 256) lens[c] = c0 + c < B ? seq_lens[c0 + c] : INT_MIN;
    __syncthreads();
    const int n4 = (min(1024, B - c0) + 3) / 4;
#pragma unroll 8
    for (int c = 0; c < n4; ++c) {
      const int4 v = lens4[c];
      const int j = c0 + 4 * c;
      rank += (v.x > L) | ((v.x == L) & (j < b));
      rank += (v.y > L) | ((v.y == L) & (j + 1 < b));
      rank += (v.z > L) | ((v.z == L) & (j + 2 < b));
      rank += (v.w > L) | ((v.w == L) & (j + 3 < b));
    }
  }
  if (b < B) order[rank] = b;
}

// ---------------------------------------------------------------------------
// Split-KV combine: o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One wave per (sequence, query, q head) output row.
// ---------------------------------------------------------------------------
template <int kD, bool kSparse>
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnArgs a) {
  const int lane = threadIdx.x;
  const int g = blockIdx.x % a.Hq;
  const int t = blockIdx.x / a.Hq;
  const int i = t % a.nq, b = t / a.nq;
  const int h = g / a.G, row = (g % a.G) * a.nq + i;
  const int seq_len = a.seq_lens[b];
  const int n_pages = seq_len > 0 ? (seq_len + kPage - 1) / kPage : 0;
  const int n_items = kSparse ? min(a.ksel, n_pages) : n_pages;
  const int per_group = split_pages(a, n_items) * a.waves_per_group;
  const int ns = (n_items + per_group - 1) / per_group;
  const size_t item0 = ((size_t)b * a.Hkv + h) * a.n_groups;

  // Splits are folded 8 at a time with all their loads in flight together.
  constexpr int kBatch = 8;
  float M = kNegInf;
  float o[kD / 64] = {};
  float den = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kBatch) {
    float m[kBatch], l[kBatch], ov[kBatch][kD / 64];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const size_t r = (item0 + min(s0 + u, ns - 1)) * a.rows + row;
      m[u] = s0 + u < ns ? a.part_ml[r * 2] : kNegInf;
      l[u] = a.part_ml[r * 2 + 1];
#pragma unroll
      for (int e = 0; e < kD / 64; ++e) ov[u][e] = a.part_o[r * kD + lane + 64 * e];
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) Mb = fmaxf(Mb, m[u]);
    if (Mb == kNegInf) continue;
    const float c = __builtin_amdgcn_exp2f(M - Mb);  // rescale what was folded so far
    den *= c;
#pragma unroll
    for (int e = 0; e < kD / 64; ++e) o[e] *= c;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = __builtin_amdgcn_exp2f(m[u] - Mb);
      den += w * l[u];
#pragma unroll
      for (int e = 0; e < kD / 64; ++e) o[e] += w * ov[u][e];
    }
    M = Mb;
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const size_t obase = (((size_t)b * a.nq + i) * a.Hq + g) * kD;
#pragma unroll
  for (int e = 0; e < kD / 64; ++e) {
    const float v = o[e] * inv;
    if (a.out_bf16)
      static_cast<uint16_t*>(a.out)[obase + lane + 64 * e] = f32_to_bf16_bits(v);
    else
      static_cast<float*>(a.out)[obase + lane + 64 * e] = v;
  }
}

template <int kD, int kNB, bool kSparse>
hipError_t launch_typed(const AttnArgs& a, s3r_dtype dt, hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)a.B * a.Hkv * a.n_groups));
  if (dt == S3R_BF16) {
    const size_t lds = (size_t)a.lds_region_bytes * a.waves_per_group;
    switch (a.waves_per_group) {
      case 1: hipLaunchKernelGGL((attn_bf16_kernel<kD, kNB, kSparse, 1>), grid, dim3(64), lds, stream, a); break;
      case 2: hipLaunchKernelGGL((attn_bf16_kernel<kD, kNB, kSparse, 2>), grid, dim3(128), lds, stream, a); break;
      case 4: hipLaunchKernelGGL((attn_bf16_kernel<kD, kNB, kSparse, 4>), grid, dim3(256), lds, stream, a); break;
      case 8:
        if constexpr (bf16_waves_per_simd<kNB>() >= 2) {
          hipLaunchKernelGGL((attn_bf16_kernel<kD, kNB, kSparse, 8>), grid, dim3(512), lds, stream, a);
          break;
        }
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  } else {
    hipLaunchKernelGGL((attn_f32_kernel<kD, kNB, kSparse>), grid, dim3(64), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dt == S3R_BF16 && a.n_groups == 1) return hipSuccess;  // merged in the workgroup
  hipLaunchKernelGGL((attn_combine_kernel<kD, kSparse>), dim3((unsigned)((size_t)a.B * a.nq * a.Hq)),
                     dim3(64), 0, stream, a);
  return hipGetLastError();
}

// The one-kernel draft step with kW waves per (sequence, kv head) and kKeys
// page keys per thread in its top-k.
template <int kD, int kW, int kKeys>
hipError_t launch_score_here(const AttnArgs& a, dim3 grid, size_t lds, hipStream_t stream) {
  const dim3 block(64 * kW);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((attn_bf16_kernel<kD, 1, true, kW, kSelScoreHere, 1, kKeys>), grid, block, lds, stream, a); break;
    case 2: hipLaunchKernelGGL((attn_bf16_kernel<kD, 1, true, kW, kSelScoreHere, 2, kKeys>), grid, block, lds, stream, a); break;
    case 4: hipLaunchKernelGGL((attn_bf16_kernel<kD, 1, true, kW, kSelScoreHere, 4, kKeys>), grid, block, lds, stream, a); break;
    case 8: hipLaunchKernelGGL((attn_bf16_kernel<kD, 1, true, kW, kSelScoreHere, 8, kKeys>), grid, block, lds, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int kD>
hipError_t launch_fused_draft(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)a.B * a.Hkv * a.n_groups));
  const size_t lds = (size_t)a.list_offset + sizeof(int32_t) * a.ksel;
  if (a.score_here) {  // one group of 4 or 8 waves per (sequence, kv head)
    if (a.n_groups != 1) return hipErrorInvalidValue;
    if (a.waves_per_group == 4)
      return a.max_pages <= fused_topk_keys(4) * 256
                 ? launch_score_here<kD, 4, fused_topk_keys(4)>(a, grid, lds, stream)
                 : launch_score_here<kD, 4, kWideTopkKeys>(a, grid, lds, stream);
    if (a.waves_per_group == 8) return launch_score_here<kD, 8, fused_topk_keys(8)>(a, grid, lds, stream);
    return hipErrorInvalidValue;
  }
  // Rank and attend after the score kernel: the draft-step plan always gives it
  // eight waves, so its top-k runs on 512 threads.
  if (a.waves_per_group != 8) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_bf16_kernel<kD, 1, true, 8, kSelFromScores>), grid, dim3(512), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_groups == 1) return e;
  hipLaunchKernelGGL((attn_combine_kernel<kD, true>), dim3((unsigned)((size_t)a.B * a.nq * a.Hq)),
                     dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int kNB>
hipError_t launch_staged(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)a.B * a.Hkv * a.n_groups));
  hipLaunchKernelGGL((attn_bf16_staged_kernel<kNB, kStagedRing>), grid, dim3(64 * kNB),
                     staged_lds_bytes(a.pages_per_split), stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_groups == 1) return e;
  hipLaunchKernelGGL((attn_combine_kernel<128, false>), dim3((unsigned)((size_t)a.B * a.nq * a.Hq)),
                     dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int kD, bool kSparse>
hipError_t launch_nb(const AttnArgs& a, s3r_dtype dt, hipStream_t stream) {
  if constexpr (kD == 128 && !kSparse) {
    if (a.staged) {
      if (dt != S3R_BF16) return hipErrorInvalidValue;
      if ((a.rows + 15) / 16 != 4) return hipErrorInvalidValue;
      return launch_staged<4>(a, stream);
    }
  }
  switch ((a.rows + 15) / 16) {
    case 1: return launch_typed<kD, 1, kSparse>(a, dt, stream);
    case 2: return launch_typed<kD, 2, kSparse>(a, dt, stream);
    case 3: return launch_typed<kD, 3, kSparse>(a, dt, stream);
    case 4: return launch_typed<kD, 4, kSparse>(a, dt, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

SplitPlan plan_attention(const s3r_paged_kv& kv, int32_t n_queries, int32_t max_items, bool dense) {
  // As many splits as resident waves: 256 CUs x 4 SIMDs x (2 waves per SIMD
  // for one MFMA row block, 1 otherwise).
  // A single query (a draft step over a short selection) splits down to one
  // two-page window per wave: its few pages then spread over a workgroup's
  // waves instead of streaming through one. Multi-query splits keep 16 pages.
  const long kMinPagesPerSplit = n_queries == 1 ? 2 : 16;
  constexpr long kMaxPagesPerSplit = 4096;   // LDS window table <= 32 KB
  constexpr size_t kMaxGroupLds = 64 * 1024;
  SplitPlan p{};
  const long B = kv.num_seqs, Hkv = kv.num_kv_heads;
  const int G = kv.num_q_heads / kv.num_kv_heads;
  p.rows = G * n_queries;
  p.row_blocks = (p.rows + 15) / 16;
  // Two row blocks over few (sequence, kv head) pairs of unequal lengths (a
  // ragged batch that has drained): four times the splits, so the long
  // sequences' splits do not run on alone after the short ones finish.
  const bool few_ragged = p.row_blocks == 2 && B * Hkv < 256 && kv.total_pages_hint > 0 &&
                          4 * (long)kv.total_pages_hint < 3 * B * (long)kv.max_pages_per_seq;
  const long kTargetItems = p.row_blocks == 1 ? 2048 : (few_ragged ? 4096 : 1024);
  long total = (long)B * max_items;
  if (kv.total_pages_hint > 0 && kv.total_pages_hint < total) total = kv.total_pages_hint;
  const double avg = (double)total / (double)B;
  long want = (kTargetItems + B * Hkv - 1) / (B * Hkv);
  if (want < 1) want = 1;
  long pps = (long)((avg + want - 1) / want);
  if (pps < kMinPagesPerSplit) pps = kMinPagesPerSplit;
  pps = (pps + 1) & ~1L;
  const long cap = ((long)max_items + 1) & ~1L;
  if (pps > cap) pps = cap;
  if (pps > kMaxPagesPerSplit) pps = kMaxPagesPerSplit;
  // Dense bf16 at head dim 128 with three row blocks: each wave's region also
  // holds its K ring, after a window table of at most 8 KB.
  const bool k_ring = dense && kv.kv_dtype == S3R_BF16 && kv.head_dim == 128 && p.row_blocks == 3;
  if (k_ring && pps > 1024) pps = 1024;
  p.pages_per_split = (int32_t)pps;
  p.n_splits = (int32_t)((max_items + pps - 1) / pps);
  // bf16: the splits of one (sequence, kv head) run as the waves of one
  // workgroup and are merged in LDS; each wave's region holds its window table,
  // then its partial.
  const size_t table = sizeof(int) * 4 * (size_t)((pps + 1) / 2);
  const size_t partial = sizeof(float) * (size_t)p.rows * (kv.head_dim + 2);
  p.lds_region_bytes = (int32_t)(((table > partial ? table : partial) + 15) & ~(size_t)15);
  size_t max_group_lds = kMaxGroupLds;
  if (k_ring) {
    const size_t ring_end = (size_t)k_ring_offset((int)pps) + kKRingBytes;
    p.lds_region_bytes = (int32_t)(((ring_end > partial ? ring_end : partial) + 255) & ~(size_t)255);
    max_group_lds = 160 * 1024;
  }
  int w = 1;
  if (kv.kv_dtype == S3R_BF16) {
    const int wmax = p.row_blocks == 1 ? 8 : 4;
    while (w < wmax && w < p.n_splits) w *= 2;
    while (w > 1 && (size_t)w * p.lds_region_bytes > max_group_lds) w /= 2;
  }
  // Dense bf16, head dim 128, four row blocks: one split per workgroup, K/V
  // staged through LDS.
  if (dense && kv.kv_dtype == S3R_BF16 && kv.head_dim == 128 && p.row_blocks == 4) {
    p.staged = 1;
    w = 1;
    p.lds_region_bytes = 0;
  }
  p.waves_per_group = w;
  p.n_groups = (p.n_splits + w - 1) / w;
  const bool global_combine = kv.kv_dtype != S3R_BF16 || p.n_groups > 1;
  const size_t items = (size_t)B * Hkv * p.n_groups;
  p.workspace_bytes = global_combine ? items * p.rows * ((size_t)kv.head_dim + 2) * sizeof(float) : 0;
  return p;
}

hipError_t launch_attention(const AttnArgs& a, s3r_dtype kv_dtype, hipStream_t stream) {
  if (a.order != nullptr) {
    hipLaunchKernelGGL(order_by_length_kernel, dim3((unsigned)((a.B + 255) / 256)), dim3(256), 0,
                       stream, a.seq_lens, a.B, a.order);
    if (hipError_t e = hipGetLastError()) return e;
  }
  if (a.scores != nullptr || a.score_here) {  // fused draft step: bf16, one row block
    if (kv_dtype != S3R_BF16 || a.rows > 16) return hipErrorInvalidValue;
    return a.D == 128 ? launch_fused_draft<128>(a, stream) : launch_fused_draft<64>(a, stream);
  }
  const bool sparse = a.sel != nullptr;
  if (a.D == 128)
    return sparse ? launch_nb<128, true>(a, kv_dtype, stream) : launch_nb<128, false>(a, kv_dtype, stream);
  if (a.D == 64)
    return sparse ? launch_nb<64, true>(a, kv_dtype, stream) : launch_nb<64, false>(a, kv_dtype, stream);
  return hipErrorInvalidValue;
}

}  // namespace s3r
