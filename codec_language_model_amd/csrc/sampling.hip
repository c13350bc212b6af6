// Per-row token choice and speculative verification.
//
// sample_or_argmax (TontaubeV1: later stages decode at temperature zero;
// Section 3.3: logits outside the stage's vocabulary are masked at sampling):
// one 256-thread workgroup per row.  Greedy rows take a block argmax (lowest
// index on ties).  Sampled rows compute z = logit / T, e = exp(z - max z) and
// draw by inverse CDF at the supplied uniform.
//
// spec_verify (Optimizing Streaming Text-to-Speech Models ..., "Speculative
// Decoding for Acoustic Tokens"): one workgroup per stream walks its K drafted
// positions in order: row normaliser, accept test u < p[x]/q[x], and on the
// first rejection an inverse-CDF draw from max(p - q, 0).
//
// The inverse CDF is deterministic and exact about where it cuts: the row is
// split into rounds of 1024 entries (256 threads x 4 consecutive entries); the
// first pass scans every round (wave prefix sums, per-wave totals in LDS); the
// running round totals locate the round that holds u*S, and a second pass
// re-derives the same prefix sums for that round only, so every interval
// bound the search compares against is one number computed once.  All
// reductions combine in a fixed order, so results do not vary run to run.
#include "clm_device.h"
#include "clm_launch.h"

namespace clm {
namespace {

constexpr int kT = 256;
constexpr int kRound = 1024;
constexpr int kMaxRounds = 1024;  // V <= 1<<20

struct Scratch {
  float wt[4][kMaxRounds];
  float rf[4];
  int ri[4];
  int pick, round;
  float target, total;
};

__device__ __forceinline__ float block_sum(float x, Scratch& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  x = wave_sum(x);
  __syncthreads();
  if (lane == 0) sc.rf[w] = x;
  __syncthreads();
  return ((sc.rf[0] + sc.rf[1]) + sc.rf[2]) + sc.rf[3];
}

__device__ __forceinline__ float block_max(float x, Scratch& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  x = wave_max(x);
  __syncthreads();
  if (lane == 0) sc.rf[w] = x;
  __syncthreads();
  return fmaxf(fmaxf(sc.rf[0], sc.rf[1]), fmaxf(sc.rf[2], sc.rf[3]));
}

__device__ __forceinline__ int block_max_int(int x, Scratch& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off, 64));
  __syncthreads();
  if (lane == 0) sc.ri[w] = x;
  __syncthreads();
  return max(max(sc.ri[0], sc.ri[1]), max(sc.ri[2], sc.ri[3]));
}

// Lowest index of the largest value among x[0:n].  Each thread scans its
// entries in increasing index order (strict >, so its first occurrence wins),
// then (value, index) pairs are reduced with ties going to the lower index.
// When the row is 16-byte aligned the scan reads float4s, eight of them in
// flight per thread before any is compared, so a row streams at memory rate.
__device__ int block_argmax(const float* __restrict__ x, int n, Scratch& sc) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  int done = 0;
  if ((reinterpret_cast<uintptr_t>(x) & 15) == 0) {
    constexpr int U = 8;
    const int n4 = n >> 2;
    const float4* __restrict__ x4 = reinterpret_cast<const float4*>(x);
    for (int j0 = 0; j0 < n4; j0 += kT * U) {
      float4 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int j = j0 + k * kT + tid;
        v[k] = j < n4 ? x4[j] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int i = (j0 + k * kT + tid) * 4;
        if (v[k].x > bv) { bv = v[k].x; bi = i; }
        if (v[k].y > bv) { bv = v[k].y; bi = i + 1; }
        if (v[k].z > bv) { bv = v[k].z; bi = i + 2; }
        if (v[k].w > bv) { bv = v[k].w; bi = i + 3; }
      }
    }
    done = n4 * 4;
  }
  for (int i = done + tid; i < n; i += kT) {
    const float v = x[i];
    if (v > bv) { bv = v; bi = i; }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(bv, off, 64);
    const int oi = __shfl_xor(bi, off, 64);
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
  }
  __syncthreads();
  if (lane == 0) { sc.rf[w] = bv; sc.ri[w] = bi; }
  __syncthreads();
  bv = sc.rf[0];
  bi = sc.ri[0];
  for (int i = 1; i < 4; ++i)
    if (sc.rf[i] > bv || (sc.rf[i] == bv && sc.ri[i] < bi)) { bv = sc.rf[i]; bi = sc.ri[i]; }
  return bi == 0x7fffffff ? 0 : bi;
}

// Largest of x[0:n], with the same float4 streaming as block_argmax.
__device__ float block_row_max(const float* __restrict__ x, int n, Scratch& sc) {
  float mx = -INFINITY;
  int done = 0;
  if ((reinterpret_cast<uintptr_t>(x) & 15) == 0) {
    constexpr int U = 8;
    const int n4 = n >> 2;
    const float4* __restrict__ x4 = reinterpret_cast<const float4*>(x);
    for (int j0 = 0; j0 < n4; j0 += kT * U) {
      float4 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int j = j0 + k * kT + threadIdx.x;
        v[k] = j < n4 ? x4[j] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      }
#pragma unroll
      for (int k = 0; k < U; ++k) mx = fmaxf(mx, fmaxf(fmaxf(v[k].x, v[k].y), fmaxf(v[k].z, v[k].w)));
    }
    done = n4 * 4;
  }
  for (int i = done + threadIdx.x; i < n; i += kT) mx = fmaxf(mx, x[i]);
  return block_max(mx, sc);
}

// min{ i : u*S < w_0 + ... + w_i } over i < n for the weights wf(i) >= 0, S
// their total; the last index with w_i > 0 if rounding leaves none; -1 if
// every weight is zero.
template <class WF>
__device__ int block_inverse_cdf(int n, float u, const WF& wf, Scratch& sc) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nrounds = (n + kRound - 1) / kRound;
  __syncthreads();
  for (int k = 0; k < nrounds; ++k) {
    const int i0 = k * kRound + tid * 4;
    float e = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i0 + i < n) e += wf(i0 + i);
    const float incl = wave_incl_scan(e, lane);
    if (lane == 63) sc.wt[w][k] = incl;
  }
  __syncthreads();
  if (tid == 0) {
    float S = 0.f;
    for (int k = 0; k < nrounds; ++k) S += ((sc.wt[0][k] + sc.wt[1][k]) + sc.wt[2][k]) + sc.wt[3][k];
    const float target = u * S;
    float C = 0.f;
    int kstar = -1;
    float before = 0.f;
    for (int k = 0; k < nrounds; ++k) {
      const float Cn = C + (((sc.wt[0][k] + sc.wt[1][k]) + sc.wt[2][k]) + sc.wt[3][k]);
      if (target < Cn) { kstar = k; before = C; break; }
      C = Cn;
    }
    sc.round = kstar;
    sc.target = target - before;
    sc.total = S;
    sc.pick = -1;
  }
  __syncthreads();
  if (!(sc.total > 0.f)) return -1;
  const int kstar = sc.round;
  if (kstar >= 0) {
    const int i0 = kstar * kRound + tid * 4;
    float ev[4];
    float e = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ev[i] = (i0 + i < n) ? wf(i0 + i) : 0.f;
      e += ev[i];
    }
    const float incl = wave_incl_scan(e, lane);
    float excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.f;
    float base = 0.f;
    for (int i = 0; i < w; ++i) base += sc.wt[i][kstar];
    const float start = base + excl, end = base + incl;
    const float tgt = sc.target;
    if (e > 0.f && start <= tgt && tgt < end) {
      float run = start;
      int pick = -1, lastpos = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        run += ev[i];
        if (ev[i] > 0.f) {
          lastpos = i;
          if (pick < 0 && tgt < run) pick = i;
        }
      }
      sc.pick = i0 + (pick < 0 ? lastpos : pick);
    }
  }
  __syncthreads();
  const int pick = sc.pick;
  if (pick >= 0) return pick;
  int last = -1;
  for (int i = tid; i < n; i += kT)
    if (wf(i) > 0.f) last = i;
  return block_max_int(last, sc);
}

__global__ __launch_bounds__(kT) void sample_kernel(SampleArgs P) {
  __shared__ Scratch sc;
  const int r = blockIdx.x;
  const float* __restrict__ x = P.logits + (size_t)r * P.ld;
  const int n = P.vocab_valid ? clampi(P.vocab_valid[r], 1, P.V) : P.V;
  const float T = P.temperature ? P.temperature[r] : 0.f;
  int tok;
  if (!(T > 0.f)) {
    tok = block_argmax(x, n, sc);
  } else {
    const float mx = block_row_max(x, n, sc);
    const float m = mx / T;
    const float u = P.uniforms[r];
    tok = block_inverse_cdf(n, u, [&](int i) { return expf(x[i] / T - m); }, sc);
    if (tok < 0) tok = 0;
  }
  if (threadIdx.x == 0) P.tokens[r] = tok;
}

__global__ __launch_bounds__(kT) void verify_kernel(VerifyArgs P) {
  __shared__ Scratch sc;
  const int b = blockIdx.x;
  const float T = P.temperature;
  const int V = P.V;
  int emitted = 0;
  for (int i = 0; i < P.K; ++i) {
    const size_t row = (size_t)b * P.K + i;
    const float* __restrict__ x = P.target_logits + row * V;
    const float* __restrict__ q = P.draft_probs + row * V;
    const int xt = clampi(P.draft_tokens[row], 0, V - 1);
    const float qx = q[xt];
    if (T > 0.f) {
      const float mx = block_row_max(x, V, sc);
      const float m = mx / T;
      float s = 0.f;
      for (int j = threadIdx.x; j < V; j += kT) s += expf(x[j] / T - m);
      const float S = block_sum(s, sc);
      const float px = expf(x[xt] / T - m) / S;
      const bool accept = qx > 0.f && P.u_accept[row] < px / qx;
      if (accept) {
        if (threadIdx.x == 0) P.out_tokens[row] = xt;
        ++emitted;
        continue;
      }
      const float ur = P.u_resample[b];
      int tok = block_inverse_cdf(
          V, ur, [&](int j) { return fmaxf(expf(x[j] / T - m) / S - q[j], 0.f); }, sc);
      if (tok < 0) tok = block_inverse_cdf(V, ur, [&](int j) { return expf(x[j] / T - m) / S; }, sc);
      if (threadIdx.x == 0) P.out_tokens[row] = tok < 0 ? 0 : tok;
      ++emitted;
      break;
    } else {
      const int amax = block_argmax(x, V, sc);
      const bool accept = qx > 0.f && xt == amax;
      if (accept) {
        if (threadIdx.x == 0) P.out_tokens[row] = xt;
        ++emitted;
        continue;
      }
      // the residual max(onehot(amax) - q, 0) is positive only at amax (or
      // zero everywhere, then the draw is from the one-hot target): amax
      if (threadIdx.x == 0) P.out_tokens[row] = amax;
      ++emitted;
      break;
    }
  }
  for (int i = emitted + threadIdx.x; i < P.K; i += kT) P.out_tokens[(size_t)b * P.K + i] = -1;
  if (threadIdx.x == 0) P.num_emitted[b] = emitted;
}

}  // namespace

hipError_t launch_sample_or_argmax(const SampleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(sample_kernel, dim3(a.M), dim3(kT), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_spec_verify(const VerifyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(verify_kernel, dim3(a.B), dim3(kT), 0, s, a);
  return hipGetLastError();
}

}  // namespace clm
