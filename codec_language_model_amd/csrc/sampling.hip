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
// Decoding for Acoustic Tokens"): one workgroup per (stream, target row)
// decides that row's draft - accept test u < p[x]/q[x] - and, if it is
// rejected, draws its residual token from max(p - q, 0); a one-thread-per-
// stream pass then keeps the drafts before the first rejection and that
// row's residual token.
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

// A row is handled by one workgroup of NT threads: 1024 for rows longer than
// 4096 entries, 256 otherwise (fewer idle waves at each barrier).
constexpr int kCH = 16;                 // consecutive entries per thread per pass
constexpr int kMaxPasses = 64;          // V <= 1 << 20 at NT = 1024 (one pass at NT = 256)
template <int NT> struct Blk {
  static constexpr int W = NT / 64;     // waves per row
  static constexpr int PASS = NT * kCH; // entries per pass
};

// exp(x / T - mx / T) as 2^((x - mx) * c), c = log2(e) / T: one subtraction,
// one multiply and the hardware exp2 (x <= mx, so the argument is <= 0).  c
// is kept finite so that x = mx gives 2^0 = 1 at any temperature.
__device__ __forceinline__ float softmax_c(float T) { return fminf(kLog2e / T, 3.0e38f); }
__device__ __forceinline__ float softmax_w(float x, float mx, float c) {
  return __builtin_amdgcn_exp2f((x - mx) * c);
}

template <int NT>
struct Scratch {
  float wf[Blk<NT>::W];
  float once[3][Blk<NT>::W];
  int wi[Blk<NT>::W];
  float ptot[kMaxPasses];
  int pick, psel;
  float target, total;
};

// The per-wave slots of a block-wide round.  Slot 0 (sc.wf) is reused, so a
// round on it first waits at a barrier for the previous round's readers;
// slots 1..3 are each used by at most one round of a kernel and skip that
// barrier, leaving one barrier per round.
template <int S, int NT>
__device__ __forceinline__ float* round_slot(Scratch<NT>& sc) {
  if constexpr (S == 0) {
    __syncthreads();
    return sc.wf;
  } else {
    return sc.once[S - 1];
  }
}

template <int NT, int S = 0>
__device__ __forceinline__ float block_max(float x, Scratch<NT>& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  x = wave_max(x);
  float* slot = round_slot<S>(sc);
  if (lane == 0) slot[w] = x;
  __syncthreads();
  float r = slot[0];
  for (int i = 1; i < Blk<NT>::W; ++i) r = fmaxf(r, slot[i]);
  return r;
}

template <int NT>
__device__ __forceinline__ int block_max_int(int x, Scratch<NT>& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  x = wave_max_i(x);
  __syncthreads();
  if (lane == 0) sc.wi[w] = x;
  __syncthreads();
  int r = sc.wi[0];
  for (int i = 1; i < Blk<NT>::W; ++i) r = max(r, sc.wi[i]);
  return r;
}

// (value, index) maximum with ties to the lower index.
template <int NT>
__device__ __forceinline__ int block_argmax_pair(float bv, int bi, Scratch<NT>& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  wave_argmax(bv, bi);
  __syncthreads();
  if (lane == 0) { sc.wf[w] = bv; sc.wi[w] = bi; }
  __syncthreads();
  bv = sc.wf[0];
  bi = sc.wi[0];
  for (int i = 1; i < Blk<NT>::W; ++i)
    if (sc.wf[i] > bv || (sc.wf[i] == bv && sc.wi[i] < bi)) { bv = sc.wf[i]; bi = sc.wi[i]; }
  return bi;
}

// Block-wide scan of the thread sums s (thread order): this thread's interval
// [start, end) of the running total, and the total.  Lane l's start is
// computed as the same expression as lane l-1's end (and a wave's base as
// the previous wave's last end), so consecutive intervals share their bound.
template <int NT, int S = 0>
__device__ __forceinline__ void block_scan(float s, float& start, float& end, float& tot, Scratch<NT>& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float incl = wave_incl_scan(s, lane);
  float prev = __shfl_up(incl, 1, 64);
  if (lane == 0) prev = 0.f;
  float* slot = round_slot<S>(sc);
  if (lane == 63) slot[w] = incl;
  __syncthreads();
  float base = 0.f, bw = 0.f;
  for (int i = 0; i < Blk<NT>::W; ++i) {
    if (i == w) bw = base;
    base += slot[i];
  }
  start = lane == 0 ? bw : bw + prev;
  end = bw + incl;
  tot = base;
}

// x[i0 .. i0+15] into v (entries at or past n get `fill`); float4 loads when
// the chunk is whole and 16-byte aligned.  Default-policy loads: the logits
// were usually written just before by the head, and reading them through the
// caches is faster than the non-temporal hint (256 x 16384: 8.5 against
// 9.5 us per call).
__device__ __forceinline__ void load16(const float* __restrict__ x, int i0, int n, float (&v)[kCH], float fill) {
  if (i0 + kCH <= n && (reinterpret_cast<uintptr_t>(x + i0) & 15) == 0) {
    const float4* p = reinterpret_cast<const float4*>(x + i0);
#pragma unroll
    for (int k = 0; k < kCH / 4; ++k) {
      const float4 f = p[k];
      v[4 * k] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < kCH; ++k) v[k] = i0 + k < n ? x[i0 + k] : fill;
  }
}

// Lowest index of the largest value among x[0:n].
template <int NT>
__device__ int row_argmax(const float* __restrict__ x, int n, Scratch<NT>& sc) {
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i0 = threadIdx.x * kCH; i0 < n; i0 += Blk<NT>::PASS) {
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
template <int NT, class WF>
__device__ int block_draw(int n, float u, const WF& wf, float (&e)[kCH], bool have, Scratch<NT>& sc) {
  constexpr int kPass = Blk<NT>::PASS;
  const int tid = threadIdx.x;
  const int npass = (n + kPass - 1) / kPass;
  float start1 = 0.f, end1 = 0.f, s1 = 0.f;   // a one-pass row keeps its interval
  for (int p = 0; p < npass; ++p) {
    if (!(have && npass == 1)) wf(p * kPass + tid * kCH, e);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kCH; ++k) s += e[k];
    float start, end, tot;
    block_scan(s, start, end, tot, sc);
    if (tid == 0) sc.ptot[p] = tot;
    start1 = start; end1 = end; s1 = s;
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
    float s = s1, start = start1, end = end1;
    if (npass > 1) {
      wf(i0, e);
      s = 0.f;
#pragma unroll
      for (int k = 0; k < kCH; ++k) s += e[k];
      float tot;
      block_scan(s, start, end, tot, sc);      // the same numbers as in the totals pass
    }
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

// block_draw for a row that fits one pass, with e already holding this
// thread's weights.  Every thread gets the scan total, so each computes the
// target u*S itself and the round in which one thread publishes it is not
// needed; the numbers compared and the token chosen are those of block_draw.
template <int NT, int S>
__device__ int block_draw_one(float u, const float (&e)[kCH], Scratch<NT>& sc) {
  const int tid = threadIdx.x;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kCH; ++k) s += e[k];
  if (tid == 0) sc.pick = -1;           // before block_scan's barriers, so before any write below
  float start, end, tot;
  block_scan<NT, S>(s, start, end, tot, sc);
  if (!(tot > 0.f)) return -1;
  const float tgt = u * tot;
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
    sc.pick = tid * kCH + (pick < 0 ? lastpos : pick);
  }
  __syncthreads();
  const int pick = sc.pick;
  if (pick >= 0) return pick;
  int last = -1;
#pragma unroll
  for (int k = 0; k < kCH; ++k)
    if (e[k] > 0.f) last = tid * kCH + k;
  return block_max_int(last, sc);
}

template <int NT>
__global__ __launch_bounds__(NT) void sample_kernel(SampleArgs P) {
  constexpr int kPass = Blk<NT>::PASS;
  __shared__ Scratch<NT> sc;
  const int r = blockIdx.x;
  const float* __restrict__ x = P.logits + (size_t)r * P.ld;
  const bool one = P.V <= kPass;
  const int t0 = threadIdx.x * kCH;
  // a row of one pass is loaded before its length and temperature arrive
  // (the row is readable up to V), so the call costs one round trip
  float v[kCH];
  if (one) load16(x, t0, P.V, v, -INFINITY);
  const int n = P.vocab_valid ? clampi(P.vocab_valid[r], 1, P.V) : P.V;
  const float T = P.temperature ? P.temperature[r] : 0.f;
  if (one) {
#pragma unroll
    for (int k = 0; k < kCH; ++k)
      if (t0 + k >= n) v[k] = -INFINITY;
  }
  int tok;
  if (!(T > 0.f)) {
    if (one) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int k = 0; k < kCH; ++k)
        if (v[k] > bv) { bv = v[k]; bi = t0 + k; }   // increasing index: first occurrence wins
      tok = block_argmax_pair(bv, bi, sc);
      if (tok == 0x7fffffff) tok = 0;
    } else {
      tok = row_argmax(x, n, sc);
    }
  } else {
    float e[kCH];
    float mx = -INFINITY;
    if (one) {
#pragma unroll
      for (int k = 0; k < kCH; ++k) mx = fmaxf(mx, v[k]);
    } else {
      for (int i0 = t0; i0 < n; i0 += kPass) {
        float y[kCH];
        load16(x, i0, n, y, -INFINITY);
#pragma unroll
        for (int k = 0; k < kCH; ++k) mx = fmaxf(mx, y[k]);
      }
    }
    mx = block_max<NT, 1>(mx, sc);
    const float c = softmax_c(T);
    const float u = P.uniforms[r];
    if (one) {
#pragma unroll
      for (int k = 0; k < kCH; ++k) e[k] = t0 + k < n ? softmax_w(v[k], mx, c) : 0.f;
      tok = block_draw_one<NT, 2>(u, e, sc);
    } else {
      auto wf = [&](int i0, float (&w)[kCH]) {
        float y[kCH];
        load16(x, i0, n, y, 0.f);
#pragma unroll
        for (int k = 0; k < kCH; ++k) w[k] = i0 + k < n ? softmax_w(y[k], mx, c) : 0.f;
      };
      tok = block_draw(n, u, wf, e, false, sc);
    }
    if (tok < 0) tok = 0;
  }
  if (threadIdx.x == 0) P.tokens[r] = tok;
}

// Sum over the block, combined in a fixed order (waves in index order).
template <int NT, int S = 0>
__device__ __forceinline__ float block_sum(float x, Scratch<NT>& sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  x = wave_sum(x);
  float* slot = round_slot<S>(sc);
  if (lane == 0) slot[w] = x;
  __syncthreads();
  float r = slot[0];
  for (int i = 1; i < Blk<NT>::W; ++i) r += slot[i];
  return r;
}

// Speculative verification, phase 1: one workgroup per (stream, target row),
// so a batch of B streams x K drafts spreads over B*K workgroups instead of
// B.  Row i < K decides its own draft: accept iff q[x] > 0 and
// u_accept < p[x] / q[x] (T = 0: iff x is the row's argmax); a rejected row
// also draws its residual token from max(p - q, 0) (from p if that is all
// zero) at u_resample, and the bonus row (i = K) draws from p.  The row's
// outcome goes into its own out_tokens slot: the drafted token (>= 0) if
// accepted, else -(token + 2), so phase 2 needs no other memory.
template <int NT>
__global__ __launch_bounds__(NT) void verify_rows_kernel(VerifyArgs P) {
  constexpr int kPass = Blk<NT>::PASS;
  __shared__ Scratch<NT> sc;
  __shared__ float s_xq[2];
  const int V = P.V, K = P.K;
  const int TK = K + P.bonus;
  const int b = blockIdx.x / TK, i = blockIdx.x - b * TK;
  const float T = P.temperature;
  const float* __restrict__ x = P.target_logits + ((size_t)b * TK + i) * V;
  const bool draft_row = i < K;
  const size_t drow = (size_t)b * K + (draft_row ? i : 0);
  const float* __restrict__ q = P.draft_probs + drow * V;
  const bool one = V <= kPass;
  const bool sampled = T > 0.f;
  const int t0 = threadIdx.x * kCH;
  // A sampled row of one pass issues all its loads at once - the row, the
  // draft row, the drafted token and the uniforms - and takes the drafted
  // entry's logit and draft probability from the registers of the thread
  // that holds them, so the row costs one round trip to memory.
  float v[kCH], qv[kCH], e[kCH];
  if (sampled && one) {
    load16(x, t0, V, v, -INFINITY);
    if (draft_row) load16(q, t0, V, qv, 0.f);
  }
  const int xt = draft_row ? clampi(P.draft_tokens[drow], 0, V - 1) : 0;
  const float ua = draft_row ? P.u_accept[drow] : 0.f;
  const float ur = P.u_resample[b];
  int result;
  if (!sampled) {
    const float qx = draft_row ? q[xt] : 0.f;
    const int amax = row_argmax(x, V, sc);
    result = (draft_row && qx > 0.f && xt == amax) ? xt : -(amax + 2);
  } else {
    float mx = -INFINITY, xx = 0.f, qx = 0.f;
    if (one) {
#pragma unroll
      for (int k = 0; k < kCH; ++k) mx = fmaxf(mx, v[k]);
      if (draft_row && xt / kCH == (int)threadIdx.x) {
        float a = 0.f, bq = 0.f;
#pragma unroll
        for (int k = 0; k < kCH; ++k)
          if (t0 + k == xt) { a = v[k]; bq = qv[k]; }
        s_xq[0] = a;
        s_xq[1] = bq;
      }
    } else {
      if (draft_row) { xx = x[xt]; qx = q[xt]; }
      for (int i0 = t0; i0 < V; i0 += kPass) {
        float y[kCH];
        load16(x, i0, V, y, -INFINITY);
#pragma unroll
        for (int k = 0; k < kCH; ++k) mx = fmaxf(mx, y[k]);
      }
    }
    mx = block_max<NT, 1>(mx, sc);        // its barrier also publishes s_xq
    if (one && draft_row) { xx = s_xq[0]; qx = s_xq[1]; }
    const float c = softmax_c(T);
    float part = 0.f;
    if (one) {
#pragma unroll
      for (int k = 0; k < kCH; ++k) part += t0 + k < V ? softmax_w(v[k], mx, c) : 0.f;
    } else {
      for (int i0 = t0; i0 < V; i0 += kPass) {
        float y[kCH];
        load16(x, i0, V, y, -INFINITY);
#pragma unroll
        for (int k = 0; k < kCH; ++k) part += i0 + k < V ? softmax_w(y[k], mx, c) : 0.f;
      }
    }
    const float S = block_sum<NT, 2>(part, sc);
    const float inv_s = 1.f / S;
    // every thread evaluates the accept test on the same numbers
    const bool accept = draft_row && qx > 0.f && ua < (softmax_w(xx, mx, c) / S) / qx;
    if (accept) {
      result = xt;
    } else {
      int tok = -1;
      if (one) {
        // residual weights max(p - q, 0), p = e / S; from p if all are zero
        if (draft_row) {
#pragma unroll
          for (int k = 0; k < kCH; ++k)
            e[k] = t0 + k < V ? fmaxf(softmax_w(v[k], mx, c) * inv_s - qv[k], 0.f) : 0.f;
          tok = block_draw_one<NT, 3>(ur, e, sc);
        }
        if (tok < 0) {
#pragma unroll
          for (int k = 0; k < kCH; ++k) e[k] = t0 + k < V ? softmax_w(v[k], mx, c) * inv_s : 0.f;
          tok = block_draw_one<NT, 0>(ur, e, sc);
        }
      } else {
        auto target = [&](int i0, float (&wgt)[kCH]) {
          float y[kCH];
          load16(x, i0, V, y, 0.f);
#pragma unroll
          for (int k = 0; k < kCH; ++k) wgt[k] = i0 + k < V ? softmax_w(y[k], mx, c) * inv_s : 0.f;
        };
        auto resid = [&](int i0, float (&wgt)[kCH]) {
          float y[kCH], z[kCH];
          load16(x, i0, V, y, 0.f);
          load16(q, i0, V, z, 0.f);
#pragma unroll
          for (int k = 0; k < kCH; ++k)
            wgt[k] = i0 + k < V ? fmaxf(softmax_w(y[k], mx, c) * inv_s - z[k], 0.f) : 0.f;
        };
        if (draft_row) tok = block_draw(V, ur, resid, e, false, sc);
        if (tok < 0) tok = block_draw(V, ur, target, e, false, sc);
      }
      result = -((tok < 0 ? 0 : tok) + 2);
    }
  }
  if (threadIdx.x == 0) P.out_tokens[(size_t)b * TK + i] = result;
}

// Phase 2: one thread per stream walks its rows in order: the first row with
// a negative slot was rejected (its residual token is decoded in place) and
// ends the stream; all K accepted emits K tokens, plus the decoded bonus
// draw with the bonus variant.  A rejection at the last draft also emits K
// tokens, so the bonus follows only when no row was rejected.  Later slots
// are padded with -1.
__global__ __launch_bounds__(256) void verify_chain_kernel(VerifyArgs P) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= P.B) return;
  const int K = P.K, TK = K + P.bonus;
  int32_t* out = P.out_tokens + (size_t)b * TK;
  int emitted = K;
  bool rejected = false;
  for (int i = 0; i < K; ++i) {
    const int v = out[i];
    if (v < 0) {
      out[i] = -v - 2;
      emitted = i + 1;
      rejected = true;
      break;
    }
  }
  if (!rejected && P.bonus) {
    out[K] = -out[K] - 2;
    emitted = K + 1;
  }
  for (int i = emitted; i < TK; ++i) out[i] = -1;
  P.num_emitted[b] = emitted;
}

}  // namespace

hipError_t launch_sample_or_argmax(const SampleArgs& a, hipStream_t s) {
  if (a.V <= Blk<256>::PASS) hipLaunchKernelGGL(sample_kernel<256>, dim3(a.M), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(sample_kernel<1024>, dim3(a.M), dim3(1024), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_spec_verify(const VerifyArgs& a, hipStream_t s) {
  const dim3 rows((unsigned)a.B * (unsigned)(a.K + a.bonus));
  if (a.V <= Blk<256>::PASS) hipLaunchKernelGGL(verify_rows_kernel<256>, rows, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(verify_rows_kernel<1024>, rows, dim3(1024), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verify_chain_kernel, dim3((a.B + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace clm
