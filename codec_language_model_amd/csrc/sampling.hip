// Per-row token choice and speculative verification.
//
// sample_or_argmax (TontaubeV1: later stages decode at temperature zero;
// Section 3.3: logits outside the stage's vocabulary are masked at sampling):
// one 1024-thread workgroup per row.  Greedy rows take a block argmax (lowest
// index on ties).  Sampled rows compute the softmax weights of z = logit / T,
// e = exp(z - max z), as 2^((logit - max logit) * log2(e) / T) (fp32, within a
// few ulps of the quotient form), and draw by inverse CDF at the supplied
// uniform.
//
// spec_verify (Optimizing Streaming Text-to-Speech Models ..., "Speculative
// Decoding for Acoustic Tokens"): one workgroup per stream.  The K target
// rows' normalisers are computed in parallel (one wave per row), then the
// drafted positions are walked in order - accept test u < p[x]/q[x] - and on
// the first rejection an inverse-CDF draw from max(p - q, 0) is made.
//
// The inverse CDF is deterministic and exact about where it cuts.  A row is
// taken in passes of 16384 entries; in a pass each thread holds 16
// consecutive entries in registers (one load of the row), sums their
// weights, and a block-wide scan over the thread sums gives every thread an
// interval [start, end) of the running total.  Interval ends are the very
// numbers the next interval starts from, so the intervals tile [0, S) with
// no gap or overlap; the one thread whose interval holds u*S walks its 16
// weights to find the token.  Rows longer than one pass first total every
// pass, then redo the pass that holds u*S.  All reductions combine in a
// fixed order, so results do not vary run to run.
#include "clm_device.h"
#include "clm_launch.h"

namespace clm {
namespace {

constexpr int kT = 1024;                // threads per row
constexpr int kW = kT / 64;             // waves per row
constexpr int kCH = 16;                 // consecutive entries per thread per pass
constexpr int kPass = kT * kCH;         // entries per pass
constexpr int kMaxPasses = 64;          // V <= 1 << 20
constexpr int kMaxDraft = 16;

// exp(x / T - mx / T) as 2^((x - mx) * c), c = log2(e) / T: one subtraction,
// one multiply and the hardware exp2 (x <= mx, so the argument is <= 0).  c
// is kept finite so that x = mx gives 2^0 = 1 at any temperature.
__device__ __forceinline__ float softmax_c(float T) { return fminf(kLog2e / T, 3.0e38f); }
__device__ __forceinline__ float softmax_w(float x, float mx, float c) {
  return __builtin_amdgcn_exp2f((x - mx) * c);
}

struct Scratch {
  float wf[kW];
  int wi[kW];
  float ptot[kMaxPasses];
  int pick, psel;
  float target, total;
};

__device__ __forceinline__ float block_max(float x, Scratch& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  x = wave_max(x);
  __syncthreads();                      // earlier readers of sc.wf are done
  if (lane == 0) sc.wf[w] = x;
  __syncthreads();
  float r = sc.wf[0];
  for (int i = 1; i < kW; ++i) r = fmaxf(r, sc.wf[i]);
  return r;
}

__device__ __forceinline__ int block_max_int(int x, Scratch& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  x = wave_max_i(x);
  __syncthreads();
  if (lane == 0) sc.wi[w] = x;
  __syncthreads();
  int r = sc.wi[0];
  for (int i = 1; i < kW; ++i) r = max(r, sc.wi[i]);
  return r;
}

// (value, index) maximum with ties to the lower index.
__device__ __forceinline__ int block_argmax_pair(float bv, int bi, Scratch& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  wave_argmax(bv, bi);
  __syncthreads();
  if (lane == 0) { sc.wf[w] = bv; sc.wi[w] = bi; }
  __syncthreads();
  bv = sc.wf[0];
  bi = sc.wi[0];
  for (int i = 1; i < kW; ++i)
    if (sc.wf[i] > bv || (sc.wf[i] == bv && sc.wi[i] < bi)) { bv = sc.wf[i]; bi = sc.wi[i]; }
  return bi;
}

// Block-wide scan of the thread sums s (thread order): this thread's interval
// [start, end) of the running total, and the total.  Lane l's start is
// computed as the same expression as lane l-1's end (and a wave's base as
// the previous wave's last end), so consecutive intervals share their bound.
__device__ __forceinline__ void block_scan(float s, float& start, float& end, float& tot, Scratch& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float incl = wave_incl_scan(s, lane);
  float prev = __shfl_up(incl, 1, 64);
  if (lane == 0) prev = 0.f;
  __syncthreads();
  if (lane == 63) sc.wf[w] = incl;
  __syncthreads();
  float base = 0.f, bw = 0.f;
  for (int i = 0; i < kW; ++i) {
    if (i == w) bw = base;
    base += sc.wf[i];
  }
  start = lane == 0 ? bw : bw + prev;
  end = bw + incl;
  tot = base;
}

// x[i0 .. i0+15] into v (entries at or past n get `fill`); float4 loads when
// the chunk is whole and 16-byte aligned.
__device__ __forceinline__ void load16(const float* __restrict__ x, int i0, int n, float (&v)[kCH], float fill) {
  if (i0 + kCH <= n && (reinterpret_cast<uintptr_t>(x + i0) & 15) == 0) {
    const float4* p = reinterpret_cast<const float4*>(x + i0);
#pragma unroll
    for (int k = 0; k < kCH / 4; ++k) {
      const float4 f = ld_nt(p + k);
      v[4 * k] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kCH; ++k) v[k] = i0 + k < n ? x[i0 + k] : fill;
  }
}

// Lowest index of the largest value among x[0:n].
__device__ int row_argmax(const float* __restrict__ x, int n, Scratch& sc) {
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i0 = threadIdx.x * kCH; i0 < n; i0 += kPass) {
    float v[kCH];
    load16(x, i0, n, v, -INFINITY);
#pragma unroll
    for (int k = 0; k < kCH; ++k)
      if (v[k] > bv) { bv = v[k]; bi = i0 + k; }   // increasing index: first occurrence wins
  }
  const int r = block_argmax_pair(bv, bi, sc);
  return r == 0x7fffffff ? 0 : r;
}

// min{ i : u*S < w_0 + ... + w_i } over i < n, S the total of the weights
// w >= 0, which wf(i0, e) gives for the 16 entries from i0 (0 past n); the
// last index with w_i > 0 if rounding leaves none; -1 if all are zero.  When
// the row fits one pass, `have` says e already holds this thread's weights.
template <class WF>
__device__ int block_draw(int n, float u, const WF& wf, float (&e)[kCH], bool have, Scratch& sc) {
  const int tid = threadIdx.x;
  const int npass = (n + kPass - 1) / kPass;
  for (int p = 0; p < npass; ++p) {
    if (!(have && npass == 1)) wf(p * kPass + tid * kCH, e);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kCH; ++k) s += e[k];
    float start, end, tot;
    block_scan(s, start, end, tot, sc);
    if (tid == 0) sc.ptot[p] = tot;
  }
  __syncthreads();
  if (tid == 0) {
    float S = 0.f;
    for (int p = 0; p < npass; ++p) S += sc.ptot[p];
    const float target = u * S;
    float C = 0.f, before = 0.f;
    int psel = -1;
    for (int p = 0; p < npass; ++p) {
      const float Cn = C + sc.ptot[p];
      if (target < Cn) { psel = p; before = C; break; }
      C = Cn;
    }
    sc.psel = psel;
    sc.target = target - before;
    sc.total = S;
    sc.pick = -1;
  }
  __syncthreads();
  if (!(sc.total > 0.f)) return -1;
  const int psel = sc.psel;
  if (psel >= 0) {
    const int i0 = psel * kPass + tid * kCH;
    if (npass > 1) wf(i0, e);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kCH; ++k) s += e[k];
    float start, end, tot;
    block_scan(s, start, end, tot, sc);      // the same numbers as in the totals pass
    const float tgt = sc.target;
    if (s > 0.f && start <= tgt && tgt < end) {
      float run = start;
      int pick = -1, lastpos = 0;
#pragma unroll
      for (int k = 0; k < kCH; ++k) {
        run += e[k];
        if (e[k] > 0.f) {
          lastpos = k;
          if (pick < 0 && tgt < run) pick = k;
        }
      }
      sc.pick = i0 + (pick < 0 ? lastpos : pick);
    }
  }
  __syncthreads();
  const int pick = sc.pick;
  if (pick >= 0) return pick;
  int last = -1;
  for (int p = 0; p < npass; ++p) {
    const int i0 = p * kPass + tid * kCH;
    wf(i0, e);
#pragma unroll
    for (int k = 0; k < kCH; ++k)
      if (e[k] > 0.f) last = i0 + k;
  }
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
    tok = row_argmax(x, n, sc);
  } else {
    // row maximum; a row of one pass keeps its logits in registers
    float v[kCH], e[kCH];
    float mx = -INFINITY;
    const bool one = n <= kPass;
    for (int i0 = threadIdx.x * kCH; i0 < n; i0 += kPass) {
      load16(x, i0, n, v, -INFINITY);
#pragma unroll
      for (int k = 0; k < kCH; ++k) mx = fmaxf(mx, v[k]);
    }
    mx = block_max(mx, sc);
    const float c = softmax_c(T);
    const float u = P.uniforms[r];
    auto wf = [&](int i0, float (&w)[kCH]) {
      float y[kCH];
      load16(x, i0, n, y, 0.f);
#pragma unroll
      for (int k = 0; k < kCH; ++k) w[k] = i0 + k < n ? softmax_w(y[k], mx, c) : 0.f;
    };
    if (one) {
      const int i0 = threadIdx.x * kCH;
#pragma unroll
      for (int k = 0; k < kCH; ++k) e[k] = i0 + k < n ? softmax_w(v[k], mx, c) : 0.f;
    }
    tok = block_draw(n, u, wf, e, one, sc);
    if (tok < 0) tok = 0;
  }
  if (threadIdx.x == 0) P.tokens[r] = tok;
}

// Statistics of one row, by one wave: max of x[0:n] and, when T > 0, the
// softmax normaliser sum_j exp(x_j / T - max / T); the lowest index of the
// max as well.  float4 reads when the row is 16-byte aligned.
struct RowStat { float m, sum; int amax; };

__device__ RowStat wave_row_stat(const float* __restrict__ x, int n, float T) {
  constexpr int U = 8;                       // float4 loads in flight per lane
  const int lane = threadIdx.x & 63;
  const bool vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  const int n4 = vec ? (n >> 2) : 0;
  const float4* __restrict__ x4 = reinterpret_cast<const float4*>(x);
  const float4 ninf = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int j0 = 0; j0 < n4; j0 += 64 * U) {
    float4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int j = j0 + 64 * k + lane;
      v[k] = j < n4 ? x4[j] : ninf;
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int i = 4 * (j0 + 64 * k + lane);
      if (v[k].x > bv) { bv = v[k].x; bi = i; }
      if (v[k].y > bv) { bv = v[k].y; bi = i + 1; }
      if (v[k].z > bv) { bv = v[k].z; bi = i + 2; }
      if (v[k].w > bv) { bv = v[k].w; bi = i + 3; }
    }
  }
  for (int i = 4 * n4 + lane; i < n; i += 64)
    if (x[i] > bv) { bv = x[i]; bi = i; }
  wave_argmax(bv, bi);
  RowStat r{bv, 0.f, bi == 0x7fffffff ? 0 : bi};
  if (T > 0.f) {
    const float c = softmax_c(T);
    float sum = 0.f;
    for (int j0 = 0; j0 < n4; j0 += 64 * U) {
      float4 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int j = j0 + 64 * k + lane;
        v[k] = j < n4 ? x4[j] : ninf;
      }
#pragma unroll
      for (int k = 0; k < U; ++k)
        sum += softmax_w(v[k].x, bv, c) + softmax_w(v[k].y, bv, c) + softmax_w(v[k].z, bv, c) +
               softmax_w(v[k].w, bv, c);
    }
    for (int i = 4 * n4 + lane; i < n; i += 64) sum += softmax_w(x[i], bv, c);
    r.sum = wave_sum(sum);
  }
  return r;
}

// One workgroup per stream.  (1) The K target rows' statistics in parallel,
// one wave per row, while the drafted token of each row is looked up.  (2)
// The accept chain, which needs only p[x] = exp(x[x]/T - m)/S for the
// drafted token of each row, walked in order by one lane.  (3) On the first
// rejection, the residual draw over that one row; with the bonus variant,
// when every draft is accepted, a draw from the target row after them.
__global__ __launch_bounds__(kT) void verify_kernel(VerifyArgs P) {
  __shared__ Scratch sc;
  __shared__ float s_m[kMaxDraft], s_sum[kMaxDraft];
  __shared__ int s_amax[kMaxDraft];
  __shared__ int s_first_reject, s_emitted;
  __shared__ int s_xt[kMaxDraft];
  __shared__ float s_qx[kMaxDraft], s_xx[kMaxDraft], s_ua[kMaxDraft];
  const int b = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float T = P.temperature;
  const int V = P.V, K = P.K;
  const int TK = K + P.bonus;            // target rows (and output rows) per stream

  auto lookup = [&]() {                  // the drafted token of each row and its numbers
    const size_t row = (size_t)b * K + lane;
    const int xt = clampi(P.draft_tokens[row], 0, V - 1);
    s_xt[lane] = xt;
    s_qx[lane] = P.draft_probs[row * V + xt];
    s_xx[lane] = P.target_logits[((size_t)b * TK + lane) * V + xt];
    s_ua[lane] = P.u_accept[row];
  };
  if (w < TK) {
    const RowStat st = wave_row_stat(P.target_logits + ((size_t)b * TK + w) * V, V, T);
    if (lane == 0) { s_m[w] = st.m; s_sum[w] = st.sum; s_amax[w] = st.amax; }
  } else if (w == kW - 1 && lane < K) {
    lookup();
  }
  if (TK >= kW && w == 0 && lane < K) lookup();   // every wave held a row: wave 0 looks up after
  __syncthreads();

  if (threadIdx.x == 0) {
    int rej = -1;
    for (int i = 0; i < K; ++i) {
      const int xt = s_xt[i];
      const float qx = s_qx[i];
      bool accept;
      if (T > 0.f) {
        const float px = softmax_w(s_xx[i], s_m[i], softmax_c(T)) / s_sum[i];
        accept = qx > 0.f && s_ua[i] < px / qx;
      } else {
        accept = qx > 0.f && xt == s_amax[i];
      }
      if (!accept) { rej = i; break; }
      P.out_tokens[(size_t)b * TK + i] = xt;
    }
    s_first_reject = rej;
    s_emitted = rej < 0 ? TK : rej + 1;
  }
  __syncthreads();
  const int rej = s_first_reject, emitted = s_emitted;

  if (rej >= 0) {
    const size_t row = (size_t)b * K + rej;            // draft row
    const size_t trow = (size_t)b * TK + rej;          // target row
    int tok;
    if (T > 0.f) {
      const float* __restrict__ x = P.target_logits + trow * V;
      const float* __restrict__ q = P.draft_probs + row * V;
      const float mx = s_m[rej], c = softmax_c(T), inv_s = 1.f / s_sum[rej];
      const float ur = P.u_resample[b];
      float e[kCH];
      auto resid = [&](int i0, float (&wgt)[kCH]) {
        float y[kCH], z[kCH];
        load16(x, i0, V, y, 0.f);
        load16(q, i0, V, z, 0.f);
#pragma unroll
        for (int k = 0; k < kCH; ++k) wgt[k] = i0 + k < V ? fmaxf(softmax_w(y[k], mx, c) * inv_s - z[k], 0.f) : 0.f;
      };
      tok = block_draw(V, ur, resid, e, false, sc);
      if (tok < 0) {
        auto target = [&](int i0, float (&wgt)[kCH]) {
          float y[kCH];
          load16(x, i0, V, y, 0.f);
#pragma unroll
          for (int k = 0; k < kCH; ++k) wgt[k] = i0 + k < V ? softmax_w(y[k], mx, c) * inv_s : 0.f;
        };
        tok = block_draw(V, ur, target, e, false, sc);
      }
      if (tok < 0) tok = 0;
    } else {
      // the residual max(onehot(amax) - q, 0) is positive only at amax (or
      // zero everywhere, then the draw is from the one-hot target): amax
      tok = s_amax[rej];
    }
    if (threadIdx.x == 0) P.out_tokens[trow] = tok;
  } else if (P.bonus) {
    // every draft accepted: one more token from the target row after them
    const size_t trow = (size_t)b * TK + K;
    int tok;
    if (T > 0.f) {
      const float* __restrict__ x = P.target_logits + trow * V;
      const float mx = s_m[K], c = softmax_c(T), inv_s = 1.f / s_sum[K];
      float e[kCH];
      auto target = [&](int i0, float (&wgt)[kCH]) {
        float y[kCH];
        load16(x, i0, V, y, 0.f);
#pragma unroll
        for (int k = 0; k < kCH; ++k) wgt[k] = i0 + k < V ? softmax_w(y[k], mx, c) * inv_s : 0.f;
      };
      tok = block_draw(V, P.u_resample[b], target, e, false, sc);
      if (tok < 0) tok = 0;
    } else {
      tok = s_amax[K];
    }
    if (threadIdx.x == 0) P.out_tokens[trow] = tok;
  }
  for (int i = emitted + threadIdx.x; i < TK; i += kT) P.out_tokens[(size_t)b * TK + i] = -1;
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
