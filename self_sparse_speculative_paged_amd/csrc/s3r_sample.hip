// Exact speculative sampling of one S3R round, the drafter's own (direct)
// sampling, and the acceptance rate.
//
// "S3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative Decoding",
// Abstract: a dense check plus speculative sampling leaves the drafted output
// distributed exactly as the dense policy's, whereas sampling straight from
// the sparse policy (no check) is the comparator the abstract finds unstable.
// The rule is that of the speculative decoding / speculative sampling works
// the S3R reference list cites: with p_i = softmax(target_i / T), q_i =
// softmax(draft_i / T), accept draft x_i iff u_i < p_i(x_i) / q_i(x_i); at the
// first rejection draw from norm(max(0, p_i - q_i)); if all gamma drafts are
// accepted draw a bonus token from p_gamma. A draft is accepted with
// probability alpha_i = sum_x min(p_i, q_i) = 1 - TV(p_i, q_i).
//
// Every pass is deterministic (fixed-order reductions, no float atomics):
//   stats:    per (sequence, row, 4096-token chunk) max and sum of
//             2^((x - max) log2(e) / T), the sum folded in fp64; the block that
//             holds a row's drafted token also keeps that token's logit;
//   residual: per (sequence, chunk), every block first folds the row
//             statistics and runs the accept scan itself (all blocks of a
//             sequence reach the same decision), then sums the chunk's
//             residual (or bonus) weights in fp64;
//   finalize: per sequence, locate the chunk holding u * sum(w) by an ordered
//             wave scan over the chunk sums, then the token inside it by an
//             ordered block scan over the chunk's recomputed weights.
// The drafter's draws (stats, then one draw block per row) and the acceptance
// rate (stats, per-chunk sums of min(p, q), an ordered fold) reuse the pieces.
// Uniforms: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11) at key
// (seed, 0), counter (offset, b, slot, stream); u = (word0 >> 11) * 2^-53.
// Streams: 0 accept tests, 1 residual and bonus draws, 2 the drafter's draws.
#include <limits.h>
#include <math.h>

#include <atomic>

#include "s3r_common.h"
#include "s3r_internal.h"

namespace s3r {
namespace {

constexpr int kChunk = 4096;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPerThread = kChunk / kThreads;  // tokens per thread of a chunk
constexpr float kNegInf = -__builtin_huge_valf();
constexpr double kLog2e = 1.4426950408889634;

// Philox4x64-10 round multipliers and Weyl key increments (Salmon et al.).
constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

__device__ double philox_uniform(uint64_t seed, uint64_t offset, uint64_t b, uint64_t slot,
                                 uint64_t stream) {
  uint64_t x0 = offset, x1 = b, x2 = slot, x3 = stream;
  uint64_t k0 = seed, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(kPhiloxM0, x0), lo0 = kPhiloxM0 * x0;
    const uint64_t hi1 = __umul64hi(kPhiloxM1, x2), lo1 = kPhiloxM1 * x2;
    const uint64_t y0 = hi1 ^ x1 ^ k0, y2 = hi0 ^ x3 ^ k1;
    x0 = y0;
    x1 = lo1;
    x2 = y2;
    x3 = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  return (double)(x0 >> 11) * 0x1.0p-53;
}

// What the final draw of a sequence needs from its accept scan.
struct Decision {
  double izt, izd;  // 1 / normaliser of the target and draft rows of the draw
  float mt, md;     // their max logits
  int32_t n;        // accepted drafts
  int32_t pad;
};

struct Layout {
  double* csum;    // [B][R][C] chunk sum of 2^((x - chunk max) * log2(e) / T)
  double* wsum;    // [B][C] chunk mass of the final draw's weights
  double* psum;    // [B][C] chunk mass of the target row (the zero-residual fallback)
  double* apart;   // [B][gamma][C] chunk sums of min(p, q)
  Decision* dec;   // [B]
  float* cmax;     // [B][R][C] chunk max logit
  float* probe;    // [B][R] logit at the row's drafted token
};

enum Pass { kSpecPass = 0, kDrawPass = 1, kAlphaPass = 2 };

// Carves the workspace (base == nullptr: sizing only); returns its size.
__host__ __device__ inline size_t layout_of(void* base, int pass, size_t B, size_t R, size_t C,
                                            size_t gamma, Layout* L) {
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* q = p ? p + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return q;
  };
  Layout l{};
  l.csum = reinterpret_cast<double*>(take(sizeof(double) * B * R * C));
  l.cmax = reinterpret_cast<float*>(take(sizeof(float) * B * R * C));
  if (pass == kSpecPass) {
    l.probe = reinterpret_cast<float*>(take(sizeof(float) * B * R));
    l.wsum = reinterpret_cast<double*>(take(sizeof(double) * B * C));
    l.psum = reinterpret_cast<double*>(take(sizeof(double) * B * C));
    l.dec = reinterpret_cast<Decision*>(take(sizeof(Decision) * B));
  }
  if (pass == kAlphaPass) l.apart = reinterpret_cast<double*>(take(sizeof(double) * B * gamma * C));
  if (L) *L = l;
  return off;
}

__device__ __forceinline__ Layout layout(const SampleArgs& a, int pass) {
  Layout l;
  layout_of(a.workspace, pass, a.B, a.rows, a.n_chunks, a.gamma, &l);
  return l;
}

// Row r of sequence b in the statistics pass: rows 0 .. draft_rows - 1 of the
// draft logits, then the rows of the target logits.
__device__ __forceinline__ const float* row_ptr(const SampleArgs& a, int b, int r) {
  return r < a.draft_rows ? a.draft_logits + ((size_t)b * a.draft_rows + r) * a.V
                          : a.target_logits + ((size_t)b * (a.gamma + 1) + (r - a.draft_rows)) * a.V;
}

// The chunk's tokens, coalesced: load k of thread t holds tokens
// lo + 4 * (t + kThreads * k) .. + 3 (16-byte loads when the row is 16-byte
// aligned, scalar loads otherwise). Tokens past hi read -inf.
__device__ __forceinline__ void load_strided(const float* row, int lo, int hi, float (&x)[kPerThread]) {
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
#pragma unroll
  for (int k = 0; k < kPerThread / 4; ++k) {
    const int t = lo + 4 * ((int)threadIdx.x + kThreads * k);
    if (vec && t + 3 < hi) {
      const f32x4 v = load_nt16<f32x4>(row + t);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * k + e] = v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * k + e] = t + e < hi ? row[t + e] : kNegInf;
    }
  }
}

// The same tokens, each thread owning kPerThread consecutive ones: thread t
// holds lo + kPerThread * t .. + kPerThread - 1 in token order.
__device__ __forceinline__ void load_contiguous(const float* row, int lo, int hi, float (&x)[kPerThread]) {
  const int t0 = lo + kPerThread * (int)threadIdx.x;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0 && t0 + kPerThread <= hi;
#pragma unroll
  for (int k = 0; k < kPerThread / 4; ++k) {
    if (vec) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + t0 + 4 * k);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * k + e] = v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * k + e] = t0 + 4 * k + e < hi ? row[t0 + 4 * k + e] : kNegInf;
    }
  }
}

// Wave reductions and scans on DPP (s3r_common.h): fixed orders, so every
// result is reproducible; the sums are fp64.
__device__ __forceinline__ double wave_sum_f64(double v) { return wave_sum_f64_uniform(v); }
__device__ __forceinline__ double wave_inclusive_scan(double v) { return wave_incl_scan_f64(v); }

// The exclusive prefix from an inclusive one: lane l gets lane l - 1's value,
// lane 0 gets 0. The shuffle runs on every lane: a lane that reads from a lane
// left out of the shuffle would read 0.
__device__ __forceinline__ double wave_exclusive_from(double incl) {
  const double up = __shfl_up(incl, 1, 64);
  return (threadIdx.x & 63) == 0 ? 0.0 : up;
}

// Minimum of non-negative ints, and maximum of ints >= -1, over the wave.
__device__ __forceinline__ int wave_min_i(int v) { return (int)wave_extreme_u32<false>((uint32_t)v); }
__device__ __forceinline__ int wave_max_i(int v) { return (int)wave_extreme_u32<true>((uint32_t)(v + 1)) - 1; }

// 2^v for a weight of the draw, the hardware fp32 exp2 as fp64. The chunk
// masses use the same expression for their rescale 2^((chunk max - M) ...), so
// a chunk has mass exactly when its largest token has a nonzero weight: an
// underflow cannot leave a chosen chunk without a token to draw.
__device__ __forceinline__ double weight_exp2(float v) { return (double)__builtin_amdgcn_exp2f(v); }

// Max M and Z = sum_c csum_c * 2^((cmax_c - M) * log2(e) / T) of one row's
// chunk statistics, folded by one wave in a fixed order (lane l takes chunks
// l, l + 64, ..., then a butterfly). A chunk without mass adds nothing (its
// rescale would be 0 * 2^(-inf - -inf)). Every lane returns the result.
__device__ __forceinline__ void fold_row(const float* cmax, const double* csum, int C, double cl,
                                         float& M, double& Z) {
  const int lane = threadIdx.x & 63;
  float m = kNegInf;
  for (int c = lane; c < C; c += 64) m = fmaxf(m, cmax[c]);
  m = wave_max_f32_uniform(m);
  double z = 0.0;
  for (int c = lane; c < C; c += 64) {
    const double s = csum[c];
    if (s > 0.0) z += s * weight_exp2((cmax[c] - m) * (float)cl);
  }
  M = m;
  Z = wave_sum_f64(z);
}

// ---------------------------------------------------------------------------
// Statistics pass over the (sequence, row, chunk) items, grid-stride: each
// block reduces one item while the next one's tokens are already in flight
// (no item's addresses depend on a load, so the prefetch is never waiting).
// ---------------------------------------------------------------------------
struct StatsItem {
  const float* row;
  int b, r, c, lo, hi, tok;
};

__device__ __forceinline__ StatsItem stats_item(const SampleArgs& a, int pass, int item) {
  StatsItem it;
  const int C = a.n_chunks;
  it.c = item % C;
  const int br = item / C;
  it.r = br % a.rows;
  it.b = br / a.rows;
  it.row = row_ptr(a, it.b, it.r);
  it.lo = it.c * kChunk;
  it.hi = min(a.V, it.lo + kChunk);
  // the drafted token whose logit this row's accept test reads (spec_sample)
  it.tok = -1;
  if (pass == kSpecPass && it.r < 2 * a.gamma)
    it.tok = a.draft_tokens[(size_t)it.b * a.gamma + (it.r < a.gamma ? it.r : it.r - a.gamma)];
  return it;
}

__global__ __launch_bounds__(kThreads) void stats_kernel(SampleArgs a, int pass, int n_items) {
  __shared__ float wm[2][kWaves];
  __shared__ double ws[2][kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float cl = (float)kLog2e / a.temperature;
  const Layout L = layout(a, pass);
  int item = blockIdx.x;
  if (item >= n_items) return;
  StatsItem it = stats_item(a, pass, item);
  float x[kPerThread];
  load_strided(it.row, it.lo, it.hi, x);
  for (int parity = 0;; parity ^= 1) {
    const int next = item + gridDim.x;
    StatsItem nt;
    float y[kPerThread];
    if (next < n_items) {  // uniform
      nt = stats_item(a, pass, next);
      load_strided(nt.row, nt.lo, nt.hi, y);
    }
    if (it.tok >= it.lo && it.tok < it.hi) {
      const int rel = it.tok - it.lo;
      if ((int)threadIdx.x == ((rel >> 2) & (kThreads - 1))) {
        const int j = 4 * (rel / (4 * kThreads)) + (rel & 3);
        float v = x[0];
#pragma unroll
        for (int e = 1; e < kPerThread; ++e) v = e == j ? x[e] : v;
        L.probe[(size_t)it.b * a.rows + it.r] = v;
      }
    }
    // Wave max, then every term against it (one rounding each), summed in
    // fp32 per thread and fp64 across the wave; thread 0 merges the four wave
    // partials in wave order. The LDS slots alternate between items, so one
    // barrier per item suffices.
    float m = x[0];
#pragma unroll
    for (int e = 1; e < kPerThread; ++e) m = fmaxf(m, x[e]);
    m = wave_max_f32_uniform(m);
    float sm = 0.f;
    if (m != kNegInf) {
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) sm += __builtin_amdgcn_exp2f((x[e] - m) * cl);
    }
    const double sd = wave_sum_f64((double)sm);
    if (lane == 0) {
      wm[parity][wave] = m;
      ws[parity][wave] = sd;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float M = wm[parity][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wm[parity][w]);
      double S = 0.0;
      if (M != kNegInf) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          if (wm[parity][w] != kNegInf) S += ws[parity][w] * weight_exp2((wm[parity][w] - M) * cl);
      }
      const size_t idx = ((size_t)it.b * a.rows + it.r) * a.n_chunks + it.c;
      L.cmax[idx] = M;
      L.csum[idx] = S;
    }
    if (next >= n_items) break;
    item = next;
    it = nt;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) x[e] = y[e];
  }
}

// ---------------------------------------------------------------------------
// The accept scan, in every block of a sequence: fold the round's 2 gamma + 1
// row statistics (wave w folds rows w, w + 4, ...; lane l takes chunks l,
// l + 64, ...), then test the gamma drafts in parallel (lane i of each wave
// tests draft i, so every wave reaches the decision without another barrier).
// ---------------------------------------------------------------------------
struct RoundRows {
  float M[2 * 16 + 1];
  double Z[2 * 16 + 1];
};

__device__ int round_decision(const SampleArgs& a, const Layout& L, int b, RoundRows& rr) {
  constexpr int kRowsPerWave = (2 * 16 + 1 + kWaves - 1) / kWaves;
  const int R = 2 * a.gamma + 1, C = a.n_chunks;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const double cl = kLog2e / (double)a.temperature;
  // The drafted tokens' logits and every statistic this wave folds are loaded
  // before any is used (one round trip), and the accept uniform is drawn
  // meanwhile.
  const int i = lane < a.gamma ? lane : 0;
  const double lt = L.probe[(size_t)b * R + a.gamma + i];
  const double ld = L.probe[(size_t)b * R + i];
  const double u = philox_uniform(a.seed, a.offset, b, i, 0);
  for (int c0 = 0; c0 < C; c0 += 64) {
    float cm[kRowsPerWave];
    double cs[kRowsPerWave];
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      const int r = wave + kWaves * k, c = c0 + lane;
      const bool ok = r < R && c < C;
      const size_t idx = ((size_t)b * R + (ok ? r : 0)) * C + (ok ? c : 0);
      cm[k] = ok ? L.cmax[idx] : kNegInf;
      cs[k] = ok ? L.csum[idx] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      const int r = wave + kWaves * k;
      if (r >= R) break;  // uniform
      const float M = wave_max_f32_uniform(cm[k]);
      const double Z = wave_sum_f64(cs[k] > 0.0 ? cs[k] * weight_exp2((cm[k] - M) * (float)cl) : 0.0);
      if (lane == 0) {
        if (c0 == 0) {
          rr.M[r] = M;
          rr.Z[r] = Z;
        } else {  // more than 64 chunks: fold this pass into the running values
          // A side without mass adds nothing; rescaling it would form
          // 0 * 2^(-inf - -inf) = NaN when every token so far is masked.
          const float Mn = fmaxf(rr.M[r], M);
          const double zr = rr.Z[r] > 0.0 ? rr.Z[r] * weight_exp2((rr.M[r] - Mn) * (float)cl) : 0.0;
          const double zp = Z > 0.0 ? Z * weight_exp2((M - Mn) * (float)cl) : 0.0;
          rr.Z[r] = zr + zp;
          rr.M[r] = Mn;
        }
      }
    }
  }
  __syncthreads();
  bool reject = false;
  if (lane < a.gamma) {
    const double p = exp2((lt - (double)rr.M[a.gamma + i]) * cl) / rr.Z[a.gamma + i];
    const double q = exp2((ld - (double)rr.M[i]) * cl) / rr.Z[i];
    reject = !(q > 0.0 ? (u < p / q) : (p > 0.0));
  }
  const uint64_t rej = __ballot(reject);
  return rej ? (int)__builtin_ctzll(rej) : a.gamma;
}

// Per-thread weights of the final draw from the two rows' logits.
struct DrawWeights {
  float mt, md;
  double izt, izd;
  float cl;
  int mode;  // 0: max(0, p - q); 1: p
  __device__ __forceinline__ double p_of(float xt) const { return weight_exp2((xt - mt) * cl) * izt; }
  __device__ __forceinline__ double operator()(float xt, float xd) const {
    const double p = p_of(xt);
    if (mode == 1) return p;
    const double q = weight_exp2((xd - md) * cl) * izd;
    return p > q ? p - q : 0.0;
  }
};

// Fixed-order block sum of v into thread 0's return value (others: partial).
__device__ __forceinline__ double block_sum_to_thread0(double v, double* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_f64(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += red[w];
  }
  return t;
}

// One block per (sequence, chunk): the accept scan, then the chunk's mass of
// the final draw's weights max(0, p - q) (p for the bonus), and of p.
__global__ __launch_bounds__(kThreads) void residual_kernel(SampleArgs a) {
  __shared__ RoundRows rr;
  __shared__ double red[2][kWaves];
  const int C = a.n_chunks;
  const int c = blockIdx.x % C, b = blockIdx.x / C;
  const int R = 2 * a.gamma + 1;
  const Layout L = layout(a, kSpecPass);
  const int n = round_decision(a, L, b, rr);
  const int tr = a.gamma + n, dr = n < a.gamma ? n : tr;
  const bool bonus = n == a.gamma;
  const double izt = 1.0 / rr.Z[tr], izd = 1.0 / rr.Z[dr];
  if (c == 0 && threadIdx.x == 0) {
    Decision d;
    d.izt = izt;
    d.izd = izd;
    d.mt = rr.M[tr];
    d.md = rr.M[dr];
    d.n = n;
    d.pad = 0;
    L.dec[b] = d;
  }
  const double cl = kLog2e / (double)a.temperature;
  if (bonus) {
    // w = p: the chunk's mass follows from its statistics, no logits read.
    if (threadIdx.x == 0) {
      const size_t idx = ((size_t)b * R + tr) * C + c;
      const double s = L.csum[idx];
      const double mass = s > 0.0 ? s * weight_exp2((L.cmax[idx] - rr.M[tr]) * (float)cl) * izt : 0.0;
      L.wsum[(size_t)b * C + c] = mass;
      L.psum[(size_t)b * C + c] = mass;
    }
    return;
  }
  const int lo = c * kChunk, hi = min(a.V, lo + kChunk);
  float xt[kPerThread], xd[kPerThread];
  load_strided(row_ptr(a, b, tr), lo, hi, xt);
  load_strided(row_ptr(a, b, dr), lo, hi, xd);
  DrawWeights wf{rr.M[tr], rr.M[dr], izt, izd, (float)cl, 0};
  double w = 0.0, ps = 0.0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    w += wf(xt[e], xd[e]);
    ps += wf.p_of(xt[e]);
  }
  w = block_sum_to_thread0(w, red[0]);
  ps = block_sum_to_thread0(ps, red[1]);
  if (threadIdx.x == 0) {
    L.wsum[(size_t)b * C + c] = w;
    L.psum[(size_t)b * C + c] = ps;
  }
}

// ---------------------------------------------------------------------------
// Locating u * total: first over the chunk masses (ordered wave scan, lanes
// owning contiguous chunk ranges), then inside the chosen chunk.
// ---------------------------------------------------------------------------
struct ChunkPick {
  int chunk;
  double before;  // mass of the chunks before it
  double target;  // u * total
  double total;
  bool fallback;  // rounding left no crossing: the last chunk with mass
};

template <class Mass>
__device__ ChunkPick pick_chunk(int C, double u, const Mass& mass) {
  const int lane = threadIdx.x & 63;
  const int per = (C + 63) / 64;
  const int c0 = min(C, lane * per), c1 = min(C, c0 + per);
  double own = 0.0;
  int last_pos = -1;
  for (int c = c0; c < c1; ++c) {
    const double w = mass(c);
    own += w;
    if (w > 0.0) last_pos = c;
  }
  const double incl = wave_inclusive_scan(own);
  const double excl = wave_exclusive_from(incl);
  ChunkPick pk;
  pk.total = readlane_f64(incl, 63);
  pk.target = u * pk.total;
  int chunk = INT_MAX;
  double before = 0.0, run = excl;
  for (int c = c0; c < c1; ++c) {
    const double w = mass(c);
    if (run + w > pk.target) {
      chunk = c;
      before = run;
      break;
    }
    run += w;
  }
  int best = wave_min_i(chunk);
  pk.fallback = best == INT_MAX;
  if (pk.fallback) best = max(wave_max_i(last_pos), 0);
  const uint64_t owner = __ballot(chunk == best);
  const double owner_before = readlane_f64(before, owner ? (int)__builtin_ctzll(owner) : 0);
  pk.before = pk.fallback ? 0.0 : owner_before;
  pk.chunk = best;
  return pk;
}

struct DrawShared {
  double wtot[kWaves];
  int first[kWaves];
  int last[kWaves];
  int token;
};

// The token of chunk [lo, hi) at which before + the running sum of w passes
// target, tokens in ascending order (thread t owns kPerThread consecutive
// ones; an ordered block scan gives each thread its start). If none passes,
// which only rounding between the two levels allows, or `fallback` is set,
// the chunk's last token with w > 0. Every thread calls it and gets the token.
template <class W>
__device__ int draw_in_chunk(const float* trow, const float* drow, int lo, int hi, double before,
                             double target, bool fallback, const W& wfn, DrawShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float xt[kPerThread], xd[kPerThread];
  load_contiguous(trow, lo, hi, xt);
  if (drow) {
    load_contiguous(drow, lo, hi, xd);
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) xd[e] = kNegInf;
  }
  const int t0 = lo + kPerThread * (int)threadIdx.x;
  double w[kPerThread], own = 0.0;
  int last = -1;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    w[e] = t0 + e < hi ? wfn(xt[e], xd[e]) : 0.0;
    own += w[e];
    if (w[e] > 0.0) last = t0 + e;
  }
  const double incl = wave_inclusive_scan(own);
  const double wexcl = wave_exclusive_from(incl);
  if (lane == 63) sh.wtot[wave] = incl;
  last = wave_max_i(last);
  if (lane == 0) sh.last[wave] = last;
  __syncthreads();
  double run = before;
  for (int v = 0; v < wave; ++v) run += sh.wtot[v];
  run += wexcl;
  const bool cross = !fallback && run + own > target;
  const uint64_t cm = __ballot(cross);
  if (lane == 0) sh.first[wave] = cm ? wave * 64 + (int)__builtin_ctzll(cm) : INT_MAX;
  __syncthreads();
  int first = INT_MAX, block_last = -1;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    first = min(first, sh.first[v]);
    block_last = max(block_last, sh.last[v]);
  }
  if (first == INT_MAX) return block_last;  // uniform: no thread crossed
  if ((int)threadIdx.x == first) {
    int tok = -1;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (tok < 0 && run + w[e] > target) tok = t0 + e;
      run += w[e];
    }
    sh.token = tok >= 0 ? tok : last;  // rounding inside the run: its last token with mass
  }
  __syncthreads();
  return sh.token;
}

// One block per sequence: the round's final draw and its tokens.
__global__ __launch_bounds__(kThreads) void finalize_kernel(SampleArgs a) {
  __shared__ DrawShared sh;
  const int b = blockIdx.x, C = a.n_chunks;
  const Layout L = layout(a, kSpecPass);
  const Decision d = L.dec[b];
  const int n = d.n;
  const int tr = a.gamma + n, dr = n < a.gamma ? n : tr;
  const bool bonus = n == a.gamma;
  const double u = philox_uniform(a.seed, a.offset, b, n, 1);
  const double* wsum = L.wsum + (size_t)b * C;
  const double* psum = L.psum + (size_t)b * C;
  ChunkPick pk = pick_chunk(C, u, [&](int c) { return wsum[c]; });
  const bool use_p = bonus || !(pk.total > 0.0);  // a residual without mass (rounding only): draw from p
  if (!bonus && use_p) pk = pick_chunk(C, u, [&](int c) { return psum[c]; });
  const int lo = pk.chunk * kChunk, hi = min(a.V, lo + kChunk);
  DrawWeights wf{d.mt, d.md, d.izt, d.izd, (float)(kLog2e / (double)a.temperature), use_p ? 1 : 0};
  const int token = draw_in_chunk(row_ptr(a, b, tr), use_p ? nullptr : row_ptr(a, b, dr), lo, hi,
                                  pk.before, pk.target, pk.fallback, wf, sh);
  const int lane = threadIdx.x;
  if (lane <= a.gamma) {
    a.out_tokens[(size_t)b * (a.gamma + 1) + lane] =
        lane < n ? a.draft_tokens[(size_t)b * a.gamma + lane] : (lane == n ? token : -1);
    if (lane == 0) a.num_accepted[b] = n;
  }
}

// ---------------------------------------------------------------------------
// The drafter's own draws: x[b][r] = ICDF(softmax(row / T), U(b, first_slot + r, 2)).
// One block per (sequence, row), after the statistics pass. The weights are
// 2^((x - M) log2(e) / T), unnormalised (the inverse CDF is scale-free).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void draw_kernel(SampleArgs a) {
  __shared__ DrawShared sh;
  const int r = blockIdx.x % a.rows, b = blockIdx.x / a.rows;
  const int C = a.n_chunks;
  const Layout L = layout(a, kDrawPass);
  const size_t base = ((size_t)b * a.rows + r) * C;
  const float* cmax = L.cmax + base;
  const double* csum = L.csum + base;
  const double cl = kLog2e / (double)a.temperature;
  float M;
  double Z;
  fold_row(cmax, csum, C, cl, M, Z);
  const double u = philox_uniform(a.seed, a.offset, b, (uint64_t)(a.first_slot + r), 2);
  const ChunkPick pk = pick_chunk(C, u, [&](int c) {
    const double s = csum[c];
    return s > 0.0 ? s * weight_exp2((cmax[c] - M) * (float)cl) : 0.0;
  });
  const int lo = pk.chunk * kChunk, hi = min(a.V, lo + kChunk);
  DrawWeights wf{M, 0.f, 1.0, 0.0, (float)cl, 1};
  const int token = draw_in_chunk(row_ptr(a, b, r), nullptr, lo, hi, pk.before, pk.target, pk.fallback,
                                  wf, sh);
  if (threadIdx.x == 0) a.out_tokens[(size_t)b * a.rows + r] = token;
}

// ---------------------------------------------------------------------------
// Acceptance rate: per (sequence, draft position, chunk) the fp64 sum of
// min(p, q) over the chunk, then an ordered fold over the chunks.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void alpha_kernel(SampleArgs a) {
  __shared__ float sM[2];
  __shared__ double sZ[2];
  __shared__ double red[kWaves];
  const int C = a.n_chunks;
  const int c = blockIdx.x % C;
  const int bi = blockIdx.x / C;
  const int i = bi % a.gamma, b = bi / a.gamma;
  const int wave = threadIdx.x >> 6;
  const Layout L = layout(a, kAlphaPass);
  const double cl = kLog2e / (double)a.temperature;
  const int lo = c * kChunk, hi = min(a.V, lo + kChunk);
  const int rq = i, rp = a.gamma + i;  // draft row i, target row i
  float xq[kPerThread], xp[kPerThread];
  load_strided(row_ptr(a, b, rq), lo, hi, xq);
  load_strided(row_ptr(a, b, rp), lo, hi, xp);
  if (wave < 2) {
    const size_t base = ((size_t)b * a.rows + (wave == 0 ? rq : rp)) * C;
    float M;
    double Z;
    fold_row(L.cmax + base, L.csum + base, C, cl, M, Z);
    if ((threadIdx.x & 63) == 0) {
      sM[wave] = M;
      sZ[wave] = Z;
    }
  }
  __syncthreads();
  const float mq = sM[0], mp = sM[1];
  const double izq = 1.0 / sZ[0], izp = 1.0 / sZ[1];
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const double q = (double)__builtin_amdgcn_exp2f((xq[e] - mq) * (float)cl) * izq;
    const double p = (double)__builtin_amdgcn_exp2f((xp[e] - mp) * (float)cl) * izp;
    s += p < q ? p : q;
  }
  s = block_sum_to_thread0(s, red);
  if (threadIdx.x == 0) L.apart[((size_t)b * a.gamma + i) * C + c] = s;
}

__global__ __launch_bounds__(kThreads) void alpha_fold_kernel(SampleArgs a) {
  const int bi = blockIdx.x * kThreads + threadIdx.x;
  if (bi >= a.B * a.gamma) return;
  const Layout L = layout(a, kAlphaPass);
  const double* part = L.apart + (size_t)bi * a.n_chunks;
  double s = 0.0;
  for (int c = 0; c < a.n_chunks; ++c) s += part[c];
  a.alpha[bi] = s;
}

// Resident blocks of the statistics pass: 8 per CU (its occupancy), 256 CUs.
constexpr int kStatsGrid = 8 * 256;

hipError_t launch_stats(const SampleArgs& a, int pass, hipStream_t stream) {
  const size_t items = (size_t)a.B * a.rows * a.n_chunks;
  const unsigned grid = (unsigned)(items < (size_t)kStatsGrid ? items : (size_t)kStatsGrid);
  hipLaunchKernelGGL(stats_kernel, dim3(grid), dim3(kThreads), 0, stream, a, pass, (int)items);
  return hipGetLastError();
}

// Scratch of s3r_spec_sample_noalloc: the same workspace layout, in a
// file-scope device array instead of a caller-provided buffer. Each device
// holds its own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[kStaticSampleScratchBytes];

}  // namespace

hipError_t static_sample_scratch(void** ptr) {
  // The array's device address, looked up once per device with that device
  // current (every device has its own copy at its own address). In host code
  // the array's name is only a stand-in: kernels get this address instead.
  static std::atomic<void*> cache[64];
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    cache[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

int32_t sample_chunks(int32_t vocab) { return (vocab + kChunk - 1) / kChunk; }

size_t sample_workspace_bytes(int32_t B, int32_t gamma, int32_t vocab) {
  return layout_of(nullptr, kSpecPass, B, 2 * (size_t)gamma + 1, sample_chunks(vocab), gamma, nullptr);
}

size_t draft_sample_workspace_bytes(int32_t B, int32_t rows, int32_t vocab) {
  return layout_of(nullptr, kDrawPass, B, rows, sample_chunks(vocab), 0, nullptr);
}

size_t acceptance_workspace_bytes(int32_t B, int32_t gamma, int32_t vocab) {
  return layout_of(nullptr, kAlphaPass, B, 2 * (size_t)gamma, sample_chunks(vocab), gamma, nullptr);
}

size_t sample_blocks(int32_t B, int32_t rows, int32_t vocab) {
  return (size_t)B * rows * sample_chunks(vocab);
}

hipError_t launch_sample(const SampleArgs& in, hipStream_t stream) {
  SampleArgs a = in;
  a.rows = 2 * a.gamma + 1;
  a.draft_rows = a.gamma;
  if (hipError_t e = launch_stats(a, kSpecPass, stream)) return e;
  hipLaunchKernelGGL(residual_kernel, dim3((unsigned)((size_t)a.B * a.n_chunks)), dim3(kThreads), 0, stream, a);
  if (hipError_t e = hipGetLastError()) return e;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)a.B), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_draft_sample(const SampleArgs& in, hipStream_t stream) {
  SampleArgs a = in;
  a.draft_rows = a.rows;
  a.target_logits = nullptr;
  a.draft_tokens = nullptr;
  if (hipError_t e = launch_stats(a, kDrawPass, stream)) return e;
  hipLaunchKernelGGL(draw_kernel, dim3((unsigned)((size_t)a.B * a.rows)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_acceptance(const SampleArgs& in, hipStream_t stream) {
  SampleArgs a = in;
  a.rows = 2 * a.gamma;
  a.draft_rows = a.gamma;
  a.draft_tokens = nullptr;
  if (hipError_t e = launch_stats(a, kAlphaPass, stream)) return e;
  hipLaunchKernelGGL(alpha_kernel, dim3((unsigned)((size_t)a.B * a.gamma * a.n_chunks)), dim3(kThreads), 0,
                     stream, a);
  if (hipError_t e = hipGetLastError()) return e;
  hipLaunchKernelGGL(alpha_fold_kernel, dim3((unsigned)(((size_t)a.B * a.gamma + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace s3r
