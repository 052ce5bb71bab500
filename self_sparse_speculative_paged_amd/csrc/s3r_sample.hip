// Exact speculative sampling of one S3R round.
//
// "S3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative Decoding",
// Abstract: the response is produced by full-attention verification and exact
// speculative sampling, so response groups follow the dense policy. The rule is
// that of the speculative decoding / speculative sampling works the S3R
// reference list cites: with p_i = softmax(target_i / T), q_i =
// softmax(draft_i / T), accept draft x_i iff u_i < p_i(x_i) / q_i(x_i); at the
// first rejection draw from norm(max(0, p_i - q_i)); if all gamma drafts are
// accepted draw a bonus token from p_gamma.
//
// Three passes, all deterministic (fixed-order reductions, no float atomics):
//   stats:    per (sequence, row, 4096-token chunk) max and sum of exp, the sum
//             accumulated in fp64;
//   residual: per (sequence, chunk) every block folds the row statistics, runs
//             the accept scan (identically in every block) and sums its chunk
//             of the residual (or bonus) weights in fp64;
//   finalize: per sequence, locate the chunk holding u * sum(w), then the token
//             inside it by an ordered block scan; write the round's tokens.
// Uniforms: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11) at key
// (seed, 0), counter (offset, b, slot, stream); u = (word0 >> 11) * 2^-53.
#include <math.h>

#include "s3r_common.h"
#include "s3r_internal.h"

namespace s3r {
namespace {

constexpr int kChunk = 4096;
constexpr int kThreads = 256;
constexpr int kPerThread = kChunk / kThreads;

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
  float* cmax;     // [B][R][C] chunk max logit
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
  l.cmax = reinterpret_cast<float*>(p);
  return l;
}

// Row r of sequence b: draft rows 0..gamma-1, target rows gamma..2*gamma.
__device__ __forceinline__ const float* row_ptr(const SampleArgs& a, int b, int r) {
  return r < a.gamma ? a.draft_logits + ((size_t)b * a.gamma + r) * a.V
                     : a.target_logits + ((size_t)b * (a.gamma + 1) + (r - a.gamma)) * a.V;
}

// exp((x - m) / T) with the argument formed in fp64 and rounded once to fp32.
__device__ __forceinline__ float scaled_exp(float x, double m, double inv_t) {
  return expf((float)(((double)x - m) * inv_t));
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
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int t = lo + threadIdx.x + kThreads * k;
    x[k] = t < hi ? row[t] : -__builtin_huge_valf();
    m = fmaxf(m, x[k]);
  }
  m = block_reduce_max(m, redf);
  const double inv_t = 1.0 / (double)a.temperature;
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k)
    if (lo + threadIdx.x + kThreads * k < hi) s += (double)scaled_exp(x[k], (double)m, inv_t);
  s = block_reduce_sum<double>(s, redd);
  if (threadIdx.x == 0) {
    const Layout L = layout_of(a.workspace, a.B, a.gamma, a.n_chunks);
    const size_t idx = ((size_t)b * (2 * a.gamma + 1) + r) * a.n_chunks + c;
    L.sum[idx] = s;
    L.cmax[idx] = m;
  }
}

// Per-block view of one sequence's round: row normalisers and the accept scan.
struct Round {
  double M[2 * 16 + 1];
  double Z[2 * 16 + 1];
  int n;  // accepted drafts
};

// Every thread r < 2*gamma+1 folds row r's chunk statistics in chunk order;
// thread 0 then runs the accept scan. Identical in every block that calls it.
__device__ void round_decision(const SampleArgs& a, int b, Round& rd) {
  const Layout L = layout_of(a.workspace, a.B, a.gamma, a.n_chunks);
  const int R = 2 * a.gamma + 1;
  const double inv_t = 1.0 / (double)a.temperature;
  const int r = threadIdx.x;
  if (r < R) {
    const size_t base = ((size_t)b * R + r) * a.n_chunks;
    double M = -__builtin_huge_val();
    for (int c = 0; c < a.n_chunks; ++c) M = fmax(M, (double)L.cmax[base + c]);
    double Z = 0.0;
    for (int c = 0; c < a.n_chunks; ++c) Z += L.sum[base + c] * exp(((double)L.cmax[base + c] - M) * inv_t);
    rd.M[r] = M;
    rd.Z[r] = Z;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    for (int i = 0; i < a.gamma; ++i) {
      const int x = a.draft_tokens[(size_t)b * a.gamma + i];
      const double lt = row_ptr(a, b, a.gamma + i)[x];
      const double ld = row_ptr(a, b, i)[x];
      const double p = exp((lt - rd.M[a.gamma + i]) * inv_t) / rd.Z[a.gamma + i];
      const double q = exp((ld - rd.M[i]) * inv_t) / rd.Z[i];
      const double u = philox_uniform(a.seed, a.offset, b, i, 0);
      const bool accept = q > 0.0 ? (u < p / q) : (p > 0.0);
      if (!accept) break;
      ++n;
    }
    rd.n = n;
  }
  __syncthreads();
}

// Weight of token t for the draw at slot n: max(0, p_n - q_n) on a rejection,
// p_gamma for the bonus. `p_out` receives p (the fallback when the residual
// has no mass).
__device__ __forceinline__ double draw_weight(const SampleArgs& a, const Round& rd, int b, int t,
                                              double inv_t, double* p_out) {
  const int n = rd.n;
  const int tr = a.gamma + n;
  const double p = (double)scaled_exp(row_ptr(a, b, tr)[t], rd.M[tr], inv_t) / rd.Z[tr];
  *p_out = p;
  if (n == a.gamma) return p;
  const double q = (double)scaled_exp(row_ptr(a, b, n)[t], rd.M[n], inv_t) / rd.Z[n];
  return p > q ? p - q : 0.0;
}

__global__ __launch_bounds__(kThreads) void residual_kernel(SampleArgs a) {
  __shared__ Round rd;
  __shared__ double redd[4];
  const int c = blockIdx.x, b = blockIdx.y;
  round_decision(a, b, rd);
  const double inv_t = 1.0 / (double)a.temperature;
  const int lo = c * kChunk, hi = min(a.V, lo + kChunk);
  double w = 0.0, ps = 0.0;
  for (int t = lo + threadIdx.x; t < hi; t += kThreads) {
    double p;
    w += draw_weight(a, rd, b, t, inv_t, &p);
    ps += p;
  }
  w = block_reduce_sum<double>(w, redd);
  ps = block_reduce_sum<double>(ps, redd);
  if (threadIdx.x == 0) {
    const Layout L = layout_of(a.workspace, a.B, a.gamma, a.n_chunks);
    L.wsum[(size_t)b * a.n_chunks + c] = w;
    L.psum[(size_t)b * a.n_chunks + c] = ps;
  }
}

__global__ __launch_bounds__(kThreads) void finalize_kernel(SampleArgs a) {
  __shared__ Round rd;
  __shared__ double scan[kThreads];
  __shared__ int s_chunk, s_use_p, s_fallback, s_first, s_last;
  __shared__ double s_base, s_target;
  const int b = blockIdx.x;
  round_decision(a, b, rd);
  const Layout L = layout_of(a.workspace, a.B, a.gamma, a.n_chunks);
  const double inv_t = 1.0 / (double)a.temperature;
  const int n = rd.n;
  if (threadIdx.x == 0) {
    const double u = philox_uniform(a.seed, a.offset, b, n, 1);
    const double* cs = L.wsum + (size_t)b * a.n_chunks;
    double total = 0.0;
    for (int c = 0; c < a.n_chunks; ++c) total += cs[c];
    int use_p = 0;
    if (!(total > 0.0)) {  // the residual has no mass (rounding only): draw from p
      use_p = 1;
      cs = L.psum + (size_t)b * a.n_chunks;
      total = 0.0;
      for (int c = 0; c < a.n_chunks; ++c) total += cs[c];
    }
    const double target = u * total;
    double cum = 0.0;
    int chunk = -1, last_pos = 0;
    for (int c = 0; c < a.n_chunks; ++c) {
      if (cs[c] > 0.0) last_pos = c;
      if (chunk < 0 && cum + cs[c] > target) {
        chunk = c;
        s_base = cum;
      }
      if (chunk < 0) cum += cs[c];
    }
    s_fallback = chunk < 0;
    if (chunk < 0) {
      chunk = last_pos;
      s_base = 0.0;
    }
    s_chunk = chunk;
    s_use_p = use_p;
    s_target = target;
    s_first = 0x7fffffff;
    s_last = -1;
  }
  __syncthreads();
  // Ordered scan of the chosen chunk: thread t owns tokens [lo + 16t, lo + 16t + 16).
  const int lo = s_chunk * kChunk, hi = min(a.V, lo + kChunk);
  const int t0 = min(hi, lo + kPerThread * (int)threadIdx.x), t1 = min(hi, t0 + kPerThread);
  double w[kPerThread];
  double local = 0.0;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    w[k] = 0.0;
    if (t0 + k < t1) {
      double p;
      const double r = draw_weight(a, rd, b, t0 + k, inv_t, &p);
      w[k] = s_use_p ? p : r;
      local += w[k];
    }
  }
  scan[threadIdx.x] = local;
  __syncthreads();
  if (threadIdx.x == 0) {  // exclusive prefix in token order
    double run = 0.0;
    for (int i = 0; i < kThreads; ++i) {
      const double v = scan[i];
      scan[i] = run;
      run += v;
    }
  }
  __syncthreads();
  double run = s_base + scan[threadIdx.x];
  int first = 0x7fffffff, last = -1;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    if (t0 + k < t1) {
      if (w[k] > 0.0) last = t0 + k;
      run += w[k];
      if (first == 0x7fffffff && !s_fallback && run > s_target) first = t0 + k;
    }
  }
  if (first != 0x7fffffff) atomicMin(&s_first, first);
  if (last >= 0) atomicMax(&s_last, last);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int token = s_first != 0x7fffffff ? s_first : s_last;
    int32_t* out = a.out_tokens + (size_t)b * (a.gamma + 1);
    for (int i = 0; i <= a.gamma; ++i)
      out[i] = i < n ? a.draft_tokens[(size_t)b * a.gamma + i] : (i == n ? token : -1);
    a.num_accepted[b] = n;
  }
}

}  // namespace

int32_t sample_chunks(int32_t vocab) { return (vocab + kChunk - 1) / kChunk; }

size_t sample_workspace_bytes(int32_t B, int32_t gamma, int32_t vocab) {
  const size_t C = (size_t)sample_chunks(vocab), R = 2 * (size_t)gamma + 1;
  return sizeof(double) * B * R * C + 2 * sizeof(double) * B * C + sizeof(float) * B * R * C;
}

hipError_t launch_sample(const SampleArgs& a, hipStream_t stream) {
  const int R = 2 * a.gamma + 1;
  hipLaunchKernelGGL(stats_kernel, dim3(a.n_chunks, R, a.B), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(residual_kernel, dim3(a.n_chunks, a.B), dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(finalize_kernel, dim3(a.B), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace s3r
