// Exact speculative sampling of one S3R round.
//
// "S3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative Decoding",
// Abstract: a dense check plus speculative sampling leaves the drafted output
// distributed exactly as the dense policy's. The rule is
// that of the speculative decoding / speculative sampling works the S3R
// reference list cites: with p_i = softmax(target_i / T), q_i =
// softmax(draft_i / T), accept draft x_i iff u_i < p_i(x_i) / q_i(x_i); at the
// first rejection draw from norm(max(0, p_i - q_i)); if all gamma drafts are
// accepted draw a bonus token from p_gamma.
//
// Four passes, all deterministic (fixed-order reductions, no float atomics):
//   stats:    per (sequence, row, 4096-token chunk) max and sum of exp, the sum
//             accumulated in fp64;
//   decide:   per sequence, fold the row statistics and run the accept scan;
//   residual: per (sequence, chunk) sum the chunk's residual (or bonus)
//             weights in fp64, per 16-token run and per chunk;
//   finalize: per sequence, locate the chunk holding u * sum(w), then the
//             16-token run inside it, then the token, each by an ordered wave
//             scan; write the round's tokens.
// Uniforms: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11) at key
// (seed, 0), counter (offset, b, slot, stream); u = (word0 >> 11) * 2^-53.
#include <math.h>

#include "s3r_common.h"
#include "s3r_internal.h"

namespace s3r {
namespace {

constexpr int kChunk = 4096;
constexpr int kThreads = 256;
constexpr int kPerThread = kChunk / kThreads;  // also the tokens of one residual run

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

struct Layout {
  double* sum;     // [B][R][C] chunk sum of exp((x - chunk max) / T)
  double* wsum;    // [B][C] chunk sum of the residual/bonus weights
  double* psum;    // [B][C] chunk sum of the target row's probabilities
  double* wrun;    // [B][C][kThreads] the same over each 16-token run
  double* prun;    // [B][C][kThreads]
  double* iz;      // [B][R] 1 / row normaliser, as the residual pass used it
  float* cmax;     // [B][R][C] chunk max logit
  float* rmax;     // [B][R] row max logit
  int* nacc;       // [B] accepted drafts
};

__host__ __device__ inline Layout layout_of(void* ws, int B, int gamma, int C) {
  const size_t R = 2 * (size_t)gamma + 1;
  Layout l;
  char* p = static_cast<char*>(ws);
  l.sum = reinterpret_cast<double*>(p);
  p += sizeof(double) * B * R * C;
  l.wsum = reinterpret_cast<double*>(p);
  p += sizeof(double) * B * C;
  l.psum = reinterpret_cast<double*>(p);
  p += sizeof(double) * B * C;
  l.wrun = reinterpret_cast<double*>(p);
  p += sizeof(double) * B * C * kThreads;
  l.prun = reinterpret_cast<double*>(p);
  p += sizeof(double) * B * C * kThreads;
  l.iz = reinterpret_cast<double*>(p);
  p += sizeof(double) * B * R;
  l.cmax = reinterpret_cast<float*>(p);
  p += sizeof(float) * B * R * C;
  l.rmax = reinterpret_cast<float*>(p);
  p += sizeof(float) * B * R;
  l.nacc = reinterpret_cast<int*>(p);
  return l;
}

// Row r of sequence b: draft rows 0..gamma-1, target rows gamma..2*gamma.
__device__ __forceinline__ const float* row_ptr(const SampleArgs& a, int b, int r) {
  return r < a.gamma ? a.draft_logits + ((size_t)b * a.gamma + r) * a.V
                     : a.target_logits + ((size_t)b * (a.gamma + 1) + (r - a.gamma)) * a.V;
}

// exp((x - m) / T) as 2^((x - m) * log2(e) / T): one v_exp_f32 per element.
// The argument's fp32 rounding moves each term by ~1e-7 relative at the
// magnitudes that carry mass; the sums are accumulated in fp64.
__device__ __forceinline__ float scaled_exp(float x, float m, float c_log2) {
  return __builtin_amdgcn_exp2f((x - m) * c_log2);
}

template <typename T>
__device__ T block_reduce_sum(T v, T* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) v += __shfl_xor(v, x, 64);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const T t = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return t;
}

__device__ float block_reduce_max(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) v = fmaxf(v, __shfl_xor(v, x, 64));
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const float t = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kThreads) void stats_kernel(SampleArgs a) {
  __shared__ float redf[4];
  __shared__ double redd[4];
  const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const float* row = row_ptr(a, b, r);
  const int lo = c * kChunk, hi = min(a.V, lo + kChunk);
  float x[kPerThread];
  float m = -__builtin_huge_valf();
  // Thread t owns tokens lo + 4*(t + 256*k) .. +3 (16-byte loads when the row
  // is 16-byte aligned, scalar loads otherwise).
  const bool vec = ((reinterpret_cast<uintptr_t>(row) & 15) == 0);
#pragma unroll
  for (int k = 0; k < kPerThread / 4; ++k) {
    const int t = lo + 4 * (threadIdx.x + kThreads * k);
    if (vec && t + 3 < hi) {
      const f32x4 v = load_nt16<f32x4>(row + t);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * k + e] = v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * k + e] = t + e < hi ? row[t + e] : -__builtin_huge_valf();
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) m = fmaxf(m, x[4 * k + e]);
  }
  m = block_reduce_max(m, redf);
  const float c_log2 = 1.4426950408889634f / a.temperature;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) s += scaled_exp(x[k], m, c_log2);  // -inf pads give 0
  const double sd = block_reduce_sum<double>((double)s, redd);
  if (threadIdx.x == 0) {
    const Layout L = layout_of(a.workspace, a.B, a.gamma, a.n_chunks);
    const size_t idx = ((size_t)b * (2 * a.gamma + 1) + r) * a.n_chunks + c;
    L.sum[idx] = sd;
    L.cmax[idx] = m;
  }
}

// Per-block view of one sequence's round: row normalisers and the accept scan.
struct Round {
  float M[2 * 16 + 1];    // row max logit
  double Z[2 * 16 + 1];   // sum over the row of 2^((x - M) * log2(e) / T)
  double iZ[2 * 16 + 1];
  int accept[16];
  int n;                  // accepted drafts
};

// Threads r < 2*gamma+1 fold row r's chunk statistics in chunk order; threads
// i < gamma then decide draft i (gathered logits, fp64 ratio, Philox uniform)
// and thread 0 takes the first rejection. Identical in every calling block.
__device__ void round_decision(const SampleArgs& a, int b, Round& rd) {
  const Layout L = layout_of(a.workspace, a.B, a.gamma, a.n_chunks);
  const int R = 2 * a.gamma + 1;
  const double c_log2 = 1.4426950408889634 / (double)a.temperature;
  // Wave w folds rows w, w+4, ...: lane l takes chunks l, l+64, ... and the
  // lanes are combined by a fixed butterfly (deterministic). The loads of all
  // the wave's rows are issued before any is folded.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kRowsPerWave = (2 * 16 + 1 + kThreads / 64 - 1) / (kThreads / 64);
  for (int c0 = 0; c0 == 0 || c0 < a.n_chunks; c0 += 64) {
    float cm[kRowsPerWave];
    double cs[kRowsPerWave];
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      const int r = wave + (kThreads / 64) * k;
      const int c = c0 + lane;
      const bool ok = r < R && c < a.n_chunks;
      const size_t idx = ((size_t)b * R + (ok ? r : 0)) * a.n_chunks + (ok ? c : 0);
      cm[k] = ok ? L.cmax[idx] : -__builtin_huge_valf();
      cs[k] = ok ? L.sum[idx] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      const int r = wave + (kThreads / 64) * k;
      if (r >= R) break;
      float M = cm[k];
#pragma unroll
      for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x, 64));
      double Z = cs[k] > 0.0 ? cs[k] * exp2(((double)cm[k] - (double)M) * c_log2) : 0.0;
#pragma unroll
      for (int x = 32; x >= 1; x >>= 1) Z += __shfl_xor(Z, x, 64);
      if (lane == 0) {
        if (c0 == 0) {
          rd.M[r] = M;
          rd.Z[r] = Z;
        } else {  // more than 64 chunks: fold this pass into the running values
          // A side without mass adds nothing; rescaling it would form
          // 0 * 2^(-inf - -inf) = NaN when every token so far is masked.
          const float Mn = fmaxf(rd.M[r], M);
          const double zr = rd.Z[r] > 0.0 ? rd.Z[r] * exp2(((double)rd.M[r] - Mn) * c_log2) : 0.0;
          const double zp = Z > 0.0 ? Z * exp2(((double)M - Mn) * c_log2) : 0.0;
          rd.Z[r] = zr + zp;
          rd.M[r] = Mn;
        }
        rd.iZ[r] = 1.0 / rd.Z[r];
      }
    }
  }
  __syncthreads();
  const int i = threadIdx.x;
  if (i < a.gamma) {
    const int x = a.draft_tokens[(size_t)b * a.gamma + i];
    const double lt = row_ptr(a, b, a.gamma + i)[x];
    const double ld = row_ptr(a, b, i)[x];
    const double p = exp2((lt - (double)rd.M[a.gamma + i]) * c_log2) / rd.Z[a.gamma + i];
    const double q = exp2((ld - (double)rd.M[i]) * c_log2) / rd.Z[i];
    const double u = philox_uniform(a.seed, a.offset, b, i, 0);
    rd.accept[i] = q > 0.0 ? (u < p / q) : (p > 0.0);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < a.gamma && rd.accept[n]) ++n;
    rd.n = n;
  }
  __syncthreads();
}

// One block per sequence: fold the row statistics, run the accept scan and
// store (row max, 1/normaliser, accepted count) for the two passes that follow.
__global__ __launch_bounds__(kThreads) void decide_kernel(SampleArgs a) {
  __shared__ Round rd;
  const int b = blockIdx.x;
  round_decision(a, b, rd);
  const Layout L = layout_of(a.workspace, a.B, a.gamma, a.n_chunks);
  const int R = 2 * a.gamma + 1;
  if (threadIdx.x < (unsigned)R) {
    L.rmax[(size_t)b * R + threadIdx.x] = rd.M[threadIdx.x];
    L.iz[(size_t)b * R + threadIdx.x] = rd.iZ[threadIdx.x];
  }
  if (threadIdx.x == 0) L.nacc[b] = rd.n;
}

__device__ __forceinline__ void load_decision(const SampleArgs& a, int b, Round& rd) {
  const Layout L = layout_of(a.workspace, a.B, a.gamma, a.n_chunks);
  const int R = 2 * a.gamma + 1;
  if (threadIdx.x < (unsigned)R) {
    rd.M[threadIdx.x] = L.rmax[(size_t)b * R + threadIdx.x];
    rd.iZ[threadIdx.x] = L.iz[(size_t)b * R + threadIdx.x];
  }
  if (threadIdx.x == 0) rd.n = L.nacc[b];
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void residual_kernel(SampleArgs a) {
  __shared__ Round rd;
  __shared__ double redd[4];
  const int c = blockIdx.x, b = blockIdx.y;
  load_decision(a, b, rd);
  const float c_log2 = 1.4426950408889634f / a.temperature;
  const int lo = c * kChunk, hi = min(a.V, lo + kChunk);
  const int tr = a.gamma + rd.n, dr = rd.n < a.gamma ? rd.n : tr;
  const float* trow = row_ptr(a, b, tr);
  const float* drow = row_ptr(a, b, dr);
  // Coalesced as in the stats pass: load k of thread t covers tokens
  // lo + 4 * (t + kThreads * k) .. + 3. A run of 16 consecutive tokens is then
  // four adjacent lanes of one load, folded by a fixed quad reduction.
  const bool vec = ((reinterpret_cast<uintptr_t>(trow) | reinterpret_cast<uintptr_t>(drow)) & 15) == 0;
  float xt[kPerThread], xd[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread / 4; ++k) {
    const int t = lo + 4 * (threadIdx.x + kThreads * k);
    if (vec && t + 3 < hi) {
      const f32x4 vt = load_nt16<f32x4>(trow + t);
      const f32x4 vd = load_nt16<f32x4>(drow + t);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xt[4 * k + e] = vt[e];
        xd[4 * k + e] = vd[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xt[4 * k + e] = t + e < hi ? trow[t + e] : -__builtin_huge_valf();
        xd[4 * k + e] = t + e < hi ? drow[t + e] : -__builtin_huge_valf();
      }
    }
  }
  const bool bonus = rd.n == a.gamma;
  const Layout L = layout_of(a.workspace, a.B, a.gamma, a.n_chunks);
  double* wrun = L.wrun + ((size_t)b * a.n_chunks + c) * kThreads;
  double* prun = L.prun + ((size_t)b * a.n_chunks + c) * kThreads;
  double w = 0.0, ps = 0.0;
#pragma unroll
  for (int k = 0; k < kPerThread / 4; ++k) {
    double wk = 0.0, pk = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {  // token order
      const double p = (double)scaled_exp(xt[4 * k + e], rd.M[tr], c_log2) * rd.iZ[tr];
      const double q = bonus ? 0.0 : (double)scaled_exp(xd[4 * k + e], rd.M[dr], c_log2) * rd.iZ[dr];
      wk += p > q ? p - q : 0.0;
      pk += p;
    }
    w += wk;
    ps += pk;
    wk += __shfl_xor(wk, 1, 64);
    pk += __shfl_xor(pk, 1, 64);
    wk += __shfl_xor(wk, 2, 64);
    pk += __shfl_xor(pk, 2, 64);
    if ((threadIdx.x & 3) == 0) {
      const int r = (kThreads / 4) * k + threadIdx.x / 4;  // run index inside the chunk
      wrun[r] = wk;
      prun[r] = pk;
    }
  }
  w = block_reduce_sum<double>(w, redd);
  ps = block_reduce_sum<double>(ps, redd);
  if (threadIdx.x == 0) {
    L.wsum[(size_t)b * a.n_chunks + c] = w;
    L.psum[(size_t)b * a.n_chunks + c] = ps;
  }
}

// Inclusive prefix sum over the 64 lanes of a wave, in lane order.
__device__ __forceinline__ double wave_inclusive_scan(double v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(v, d, 64);
    if (lane >= d) v += y;
  }
  return v;
}

// One wave per sequence draws the round's last token by inverse CDF over the
// residual (or bonus) weights: lanes own contiguous chunk ranges, then
// contiguous 64-token runs of the chosen chunk; running sums are ordered wave
// scans, so the draw is deterministic.
constexpr int kFinalizeLanes = 64;

__global__ __launch_bounds__(kFinalizeLanes) void finalize_kernel(SampleArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const Layout L = layout_of(a.workspace, a.B, a.gamma, a.n_chunks);
  const int R = 2 * a.gamma + 1;
  const int n = L.nacc[b];
  const int tr = a.gamma + n, dr = n < a.gamma ? n : tr;
  const float Mt = L.rmax[(size_t)b * R + tr], Md = L.rmax[(size_t)b * R + dr];
  const double iZt = L.iz[(size_t)b * R + tr], iZd = L.iz[(size_t)b * R + dr];
  const bool bonus = n == a.gamma;
  const double u = philox_uniform(a.seed, a.offset, b, n, 1);

  // Chunk level.
  const int per = (a.n_chunks + 63) / 64;
  const int c0 = min(a.n_chunks, lane * per), c1 = min(a.n_chunks, c0 + per);
  double own_w = 0.0, own_p = 0.0;
  int last_pos = -1;
  for (int c = c0; c < c1; ++c) {
    const double w = L.wsum[(size_t)b * a.n_chunks + c];
    own_w += w;
    own_p += L.psum[(size_t)b * a.n_chunks + c];
    if (w > 0.0) last_pos = c;
  }
  double incl = wave_inclusive_scan(own_w);
  double total = __shfl(incl, 63, 64);
  const bool use_p = !(total > 0.0);  // residual without mass (rounding only): draw from p
  if (use_p) {
    incl = wave_inclusive_scan(own_p);
    total = __shfl(incl, 63, 64);
  }
  const double target = u * total;
  int chunk = 0x7fffffff;
  double before = 0.0;
  {
    double run = incl - (use_p ? own_p : own_w);
    for (int c = c0; c < c1; ++c) {
      const double w = use_p ? L.psum[(size_t)b * a.n_chunks + c] : L.wsum[(size_t)b * a.n_chunks + c];
      if (use_p && w > 0.0) last_pos = c;
      if (run + w > target) {
        chunk = c;
        before = run;
        break;
      }
      run += w;
    }
  }
  // The first crossing chunk over the wave (or, if rounding left none, the
  // last chunk with mass).
  int best = chunk;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) best = min(best, __shfl_xor(best, x, 64));
  const bool fallback = best == 0x7fffffff;
  if (fallback) {
    int lp = last_pos;
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) lp = max(lp, __shfl_xor(lp, x, 64));
    best = max(lp, 0);
  }
  const unsigned long long owner = __ballot(chunk == best);
  const double base = fallback ? 0.0 : __shfl(before, owner ? __ffsll(owner) - 1 : 0, 64);

  // Run level inside the chosen chunk: lane l scans runs 4l .. 4l+3. Rounding
  // can leave the target past the runs' total; then (as for chunks) the last
  // run with mass is taken.
  const double* runs = (use_p ? L.prun : L.wrun) + ((size_t)b * a.n_chunks + best) * kThreads;
  double rw[kThreads / 64], rown = 0.0;
#pragma unroll
  for (int e = 0; e < kThreads / 64; ++e) {
    rw[e] = runs[(kThreads / 64) * lane + e];
    rown += rw[e];
  }
  const double rincl = wave_inclusive_scan(rown);
  double rrun = base + rincl - rown;
  int rfirst = 0x7fffffff, rlast = -1;
  double rbefore = 0.0;
#pragma unroll
  for (int e = 0; e < kThreads / 64; ++e) {
    const int r = (kThreads / 64) * lane + e;
    if (rw[e] > 0.0) rlast = r;
    if (rfirst == 0x7fffffff && !fallback && rrun + rw[e] > target) {
      rfirst = r;
      rbefore = rrun;
    }
    rrun += rw[e];
  }
  int rsel = rfirst;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) rsel = min(rsel, __shfl_xor(rsel, x, 64));
  const bool rfall = rsel == 0x7fffffff;
  if (rfall) {
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) rlast = max(rlast, __shfl_xor(rlast, x, 64));
    rsel = max(rlast, 0);
  }
  const unsigned long long rowner = __ballot(rfirst == rsel);
  const double rbase = rfall ? 0.0 : __shfl(rbefore, rowner ? __ffsll(rowner) - 1 : 0, 64);

  // Token level: lanes 0..15 take the run's 16 tokens.
  const float c_log2 = 1.4426950408889634f / a.temperature;
  const int lo = best * kChunk, hi = min(a.V, lo + kChunk);
  const int t = lo + kPerThread * rsel + (lane & (kPerThread - 1));
  const bool mine = lane < kPerThread && t < hi;
  const float* trow = row_ptr(a, b, tr);
  const float* drow = row_ptr(a, b, dr);
  const float xt = mine ? trow[t] : -__builtin_huge_valf();
  const float xd = mine ? drow[t] : -__builtin_huge_valf();
  const double p = (double)scaled_exp(xt, Mt, c_log2) * iZt;
  const double q = bonus ? 0.0 : (double)scaled_exp(xd, Md, c_log2) * iZd;
  const double w = mine ? (use_p ? p : (p > q ? p - q : 0.0)) : 0.0;
  const double tincl = wave_inclusive_scan(w);
  const bool hit = mine && !fallback && !rfall && rbase + tincl > target;
  int first = hit ? t : 0x7fffffff;
  int last = mine && w > 0.0 ? t : -1;
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) {
    first = min(first, __shfl_xor(first, x, 64));
    last = max(last, __shfl_xor(last, x, 64));
  }
  if (lane <= a.gamma) {
    const int token = first != 0x7fffffff ? first : last;
    a.out_tokens[(size_t)b * (a.gamma + 1) + lane] =
        lane < n ? a.draft_tokens[(size_t)b * a.gamma + lane] : (lane == n ? token : -1);
    if (lane == 0) a.num_accepted[b] = n;
  }
}

}  // namespace

int32_t sample_chunks(int32_t vocab) { return (vocab + kChunk - 1) / kChunk; }

size_t sample_workspace_bytes(int32_t B, int32_t gamma, int32_t vocab) {
  const size_t C = (size_t)sample_chunks(vocab), R = 2 * (size_t)gamma + 1;
  return sizeof(double) * B * R * C + 2 * sizeof(double) * B * C +
         2 * sizeof(double) * B * C * kThreads + sizeof(double) * B * R +
         sizeof(float) * B * R * C + sizeof(float) * B * R + sizeof(int) * B;
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t stream) {
  const int R = 2 * a.gamma + 1;
  hipLaunchKernelGGL(stats_kernel, dim3(a.n_chunks, R, a.B), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decide_kernel, dim3(a.B), dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(residual_kernel, dim3(a.n_chunks, a.B), dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(finalize_kernel, dim3(a.B), dim3(kFinalizeLanes), 0, stream, a);
  return hipGetLastError();
}

}  // namespace s3r
