// Split-KV flash-decode attention over a paged, ragged KV cache (gfx950).
//
// What it computes (TTS Serving, in depth, "Token generation under a frame
// budget": each decode step reads the stream's KV cache; Optimizing Streaming
// Text-to-Speech Models ..., "Speculative Decoding for Acoustic Tokens": a
// causal block of K queries scores K drafted positions in one pass):
//   o[b,j,h] = softmax(scale * q[b,j,h] . K[0:n_j, h/G]) . V[0:n_j, h/G],
//   n_j = kv_len[b] - (Kq-1-j).
//
// Work decomposition.  A work item is (stream b, KV head h, split s): the
// tokens [s*split, min((s+1)*split, kv_len[b])) of one KV head.  All G*Kq
// query rows that share the KV head are served by the one pass over its
// K/V bytes, so every K/V byte is read from HBM once per step.  The grid is
// persistent: every workgroup derives the item list from kv_len (a prefix sum
// of per-stream split counts, in LDS) and strides through it, so no workgroup
// is launched for splits past a stream's end.
//
// Inside an item the 4 waves take 16-token tiles round-robin.  In a tile a
// wave reads the keys as 16-byte loads, LPR lanes per key row (one 256-byte
// row per 16 lanes for bf16, D = 128), so each load instruction covers whole
// rows contiguously; the LPR partial dot products are summed with DPP inside
// the 16-lane row.  Values are stored transposed inside a block ([D][bs]), so
// a lane reads, for each of its head dimensions, the run of keys its group
// scored - again contiguous across the wave.  Each key group keeps its own
// online-softmax state (running max m, sum l, accumulator) in registers; the
// groups of a wave are merged with shuffles, the waves through LDS, and the
// splits of a (b, h) by the last workgroup to finish it, in split order.
#include "clm_device.h"
#include "clm_launch.h"

namespace clm {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxB = 4096;
constexpr long kMaxCounters = 65536;  // completion counters: one per (stream, KV head)

template <int BYTES> struct VecT;
template <> struct VecT<4> { using type = uint32_t; };
template <> struct VecT<8> { using type = uint2; };
template <> struct VecT<16> { using type = uint4; };

template <typename T, int D>
struct Geo {
  static constexpr int ESZ = (int)sizeof(T);
  static constexpr int VE = 16 / ESZ;                    // elements per 16-byte chunk
  static constexpr int CHUNKS = D / VE;                  // chunks per key row
  static constexpr int LPR = CHUNKS > 16 ? 16 : CHUNKS;  // lanes sharing one key row
  static constexpr int CPL = CHUNKS / LPR;               // chunks per lane per key
  static constexpr int NG = 64 / LPR;                    // key groups per wave
  static constexpr int KPG = 16 / NG;                    // keys per group per tile
  static constexpr int DPL = D / LPR;                    // head dims per lane in P.V
  static constexpr int VBYTES = KPG * ESZ;               // V bytes per lane per dim
  using VT = typename VecT<VBYTES>::type;
};

__device__ __forceinline__ void unpack_v(uint32_t w, float* f, uint16_t) {
  f[0] = bf16_lo(w);
  f[1] = bf16_hi(w);
}
__device__ __forceinline__ void unpack_v(uint2 w, float* f, uint16_t) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
}
__device__ __forceinline__ void unpack_v(uint4 w, float* f, float) {
  f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
  f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
}

// Partial dot product of one 16-byte chunk of q with one of k.
__device__ __forceinline__ float chunk_dot(const uint32_t* qw, uint4 k, float acc, uint16_t) {
  acc = dot2_bf16(qw[0], k.x, acc);
  acc = dot2_bf16(qw[1], k.y, acc);
  acc = dot2_bf16(qw[2], k.z, acc);
  acc = dot2_bf16(qw[3], k.w, acc);
  return acc;
}
__device__ __forceinline__ float chunk_dot(const uint32_t* qw, uint4 k, float acc, float) {
  acc = fmaf(__uint_as_float(qw[0]), __uint_as_float(k.x), acc);
  acc = fmaf(__uint_as_float(qw[1]), __uint_as_float(k.y), acc);
  acc = fmaf(__uint_as_float(qw[2]), __uint_as_float(k.z), acc);
  acc = fmaf(__uint_as_float(qw[3]), __uint_as_float(k.w), acc);
  return acc;
}

__device__ __forceinline__ void store_out(uint16_t* p, float x) { *p = f32_to_bf16(x); }
__device__ __forceinline__ void store_out(float* p, float x) { *p = x; }

struct KParams {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* block_table;
  const int32_t* kv_len;
  void* o;
  int* counters;
  float* part_ml;   // [B][H_kv][max_splits][NR][2]
  float* part_acc;  // [B][H_kv][max_splits][NR][D]
  int max_blocks, cap, B, Kq, H_q, H_kv, G, nr, bs, num_blocks, split, max_splits;
  float scale_log2;
};

template <typename T, int D>
__device__ __forceinline__ int split_count(int len, const KParams& P) {
  int n = clampi(len, 1, P.cap);
  int s = (n + P.split - 1) / P.split;
  return clampi(s, 1, P.max_splits);
}

template <typename T, int D, int NR>
__global__ __launch_bounds__(kThreads) void decode_attention_kernel(KParams P) {
  using G_ = Geo<T, D>;
  constexpr int LPR = G_::LPR, CPL = G_::CPL, KPG = G_::KPG, DPL = G_::DPL, VE = G_::VE;
  using VT = typename G_::VT;

  __shared__ int s_prefix[kMaxB + 1];
  __shared__ int s_wsum[kWaves];
  __shared__ float s_m[kWaves][NR];
  __shared__ float s_l[kWaves][NR];
  __shared__ float s_acc[kWaves][NR][D];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int g = lane / LPR;
  const int c = lane % LPR;

  const T* __restrict__ qp = static_cast<const T*>(P.q);
  const T* __restrict__ kc = static_cast<const T*>(P.kc);
  const T* __restrict__ vc = static_cast<const T*>(P.vc);
  T* __restrict__ op = static_cast<T*>(P.o);

  // ---- item list: exclusive prefix of per-stream split counts ---------------
  {
    const int per = (P.B + kThreads - 1) / kThreads;
    const int b0 = tid * per;
    int local = 0;
    for (int k = 0; k < per; ++k) {
      int b = b0 + k;
      if (b < P.B) local += split_count<T, D>(P.kv_len[b], P);
    }
    int incl = wave_incl_scan_i(local, lane);
    if (lane == 63) s_wsum[w] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < w; ++i) base += s_wsum[i];
    int run = base + incl - local;
    for (int k = 0; k < per; ++k) {
      int b = b0 + k;
      if (b < P.B) {
        s_prefix[b] = run;
        run += split_count<T, D>(P.kv_len[b], P);
      }
    }
    if (tid == 0) s_prefix[P.B] = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    __syncthreads();
  }
  const int total_items = s_prefix[P.B] * P.H_kv;

  for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
    const int u = item / P.H_kv;
    const int h = item - u * P.H_kv;
    int lo = 0, hi = P.B - 1;  // largest b with s_prefix[b] <= u
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= u) lo = mid; else hi = mid - 1;
    }
    const int b = uniform(lo);
    const int s = uniform(u - s_prefix[b]);
    const int ns = s_prefix[b + 1] - s_prefix[b];

    const int n_total = clampi(P.kv_len[b], 1, P.cap);
    const int n_min = n_total - (P.Kq - 1);       // keys seen by the first query
    const int t0 = s * P.split;
    const int t1 = min(t0 + P.split, n_total);
    const int n_tiles = (t1 - t0 + 15) >> 4;

    // ---- this lane's slice of the query rows --------------------------------
    uint32_t qw[NR][4 * CPL];
    int n_r[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      n_r[r] = 0;
#pragma unroll
      for (int i = 0; i < 4 * CPL; ++i) qw[r][i] = 0u;
      if (r < P.nr) {
        const int j = r / P.G, gi = r - (r / P.G) * P.G;
        n_r[r] = n_total - (P.Kq - 1 - j);
        const T* qrow = qp + ((size_t)(b * P.Kq + j) * P.H_q + h * P.G + gi) * D;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
          uint4 v = *reinterpret_cast<const uint4*>(qrow + (c + cc * LPR) * VE);
          qw[r][cc * 4 + 0] = v.x; qw[r][cc * 4 + 1] = v.y;
          qw[r][cc * 4 + 2] = v.z; qw[r][cc * 4 + 3] = v.w;
        }
      }
    }

    float m[NR], l[NR], acc[NR][DPL];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      m[r] = kNegBig;
      l[r] = 0.f;
#pragma unroll
      for (int jj = 0; jj < DPL; ++jj) acc[r][jj] = 0.f;
    }

    const int32_t* bt_row = P.block_table + (size_t)b * P.max_blocks;
    auto tile_bases = [&](int ti, size_t& kb, size_t& vb) {
      const int tk = t0 + (ti << 4);
      const int blk = clampi(bt_row[tk / P.bs], 0, P.num_blocks - 1);
      const int slot0 = tk % P.bs;
      const size_t hb = (size_t)blk * P.H_kv + h;
      kb = (hb * P.bs + slot0) * D;
      vb = hb * D * P.bs + slot0;
    };

    uint4 kr[KPG][CPL];
    VT vr[DPL];
    int ti = w;
    if (ti < n_tiles) {
      size_t kb, vb;
      tile_bases(ti, kb, vb);
#pragma unroll
      for (int i = 0; i < KPG; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
          kr[i][cc] = *reinterpret_cast<const uint4*>(kc + kb + (size_t)(g * KPG + i) * D + (c + cc * LPR) * VE);
#pragma unroll
      for (int jj = 0; jj < DPL; ++jj)
        vr[jj] = *reinterpret_cast<const VT*>(vc + vb + (size_t)(c + LPR * jj) * P.bs + g * KPG);
    }

    for (; ti < n_tiles; ti += kWaves) {
      // issue the next tile's loads before computing on this one
      uint4 nk[KPG][CPL];
      VT nv[DPL];
      const int tn = ti + kWaves;
      if (tn < n_tiles) {
        size_t kb, vb;
        tile_bases(tn, kb, vb);
#pragma unroll
        for (int i = 0; i < KPG; ++i)
#pragma unroll
          for (int cc = 0; cc < CPL; ++cc)
            nk[i][cc] = *reinterpret_cast<const uint4*>(kc + kb + (size_t)(g * KPG + i) * D + (c + cc * LPR) * VE);
#pragma unroll
        for (int jj = 0; jj < DPL; ++jj)
          nv[jj] = *reinterpret_cast<const VT*>(vc + vb + (size_t)(c + LPR * jj) * P.bs + g * KPG);
      }

      const int tk = t0 + (ti << 4);
      const bool full = tk + 16 <= n_min;
      float vf[DPL][KPG];
#pragma unroll
      for (int jj = 0; jj < DPL; ++jj) unpack_v(vr[jj], vf[jj], T());
      if (!full) {
#pragma unroll
        for (int i = 0; i < KPG; ++i) {
          if (tk + g * KPG + i >= n_total) {
#pragma unroll
            for (int jj = 0; jj < DPL; ++jj) vf[jj][i] = 0.f;  // slot not written yet
          }
        }
      }

#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (r < P.nr) {
          float sc[KPG];
#pragma unroll
          for (int i = 0; i < KPG; ++i) {
            float part = 0.f;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) part = chunk_dot(&qw[r][cc * 4], kr[i][cc], part, T());
            sc[i] = group_sum<LPR>(part) * P.scale_log2;
          }
          if (!full) {
#pragma unroll
            for (int i = 0; i < KPG; ++i)
              if (tk + g * KPG + i >= n_r[r]) sc[i] = -INFINITY;
          }
          float mx = sc[0];
#pragma unroll
          for (int i = 1; i < KPG; ++i) mx = fmaxf(mx, sc[i]);
          const float m_new = fmaxf(m[r], mx);
          const float corr = __builtin_amdgcn_exp2f(m[r] - m_new);
          float p[KPG];
          float psum = 0.f;
#pragma unroll
          for (int i = 0; i < KPG; ++i) {
            p[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
            psum += p[i];
          }
          l[r] = l[r] * corr + psum;
#pragma unroll
          for (int jj = 0; jj < DPL; ++jj) {
            float a = acc[r][jj] * corr;
#pragma unroll
            for (int i = 0; i < KPG; ++i) a = fmaf(p[i], vf[jj][i], a);
            acc[r][jj] = a;
          }
          m[r] = m_new;
        }
      }

#pragma unroll
      for (int i = 0; i < KPG; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) kr[i][cc] = nk[i][cc];
#pragma unroll
      for (int jj = 0; jj < DPL; ++jj) vr[jj] = nv[jj];
    }

    // ---- merge the key groups of this wave (lanes c, c+LPR, c+2LPR, ...) -----
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (r < P.nr) {
          const float mo = __shfl_xor(m[r], off, 64);
          const float lo_ = __shfl_xor(l[r], off, 64);
          const float M = fmaxf(m[r], mo);
          const float fa = __builtin_amdgcn_exp2f(m[r] - M);
          const float fb = __builtin_amdgcn_exp2f(mo - M);
          l[r] = l[r] * fa + lo_ * fb;
#pragma unroll
          for (int jj = 0; jj < DPL; ++jj) acc[r][jj] = acc[r][jj] * fa + __shfl_xor(acc[r][jj], off, 64) * fb;
          m[r] = M;
        }
      }
    }
    if (lane < LPR) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (r < P.nr) {
#pragma unroll
          for (int jj = 0; jj < DPL; ++jj) s_acc[w][r][c + LPR * jj] = acc[r][jj];
          if (lane == 0) { s_m[w][r] = m[r]; s_l[w][r] = l[r]; }
        }
      }
    }
    __syncthreads();

    // ---- merge the 4 waves; finish or publish the split ------------------------
    const size_t bh = (size_t)b * P.H_kv + h;
    for (int e = tid; e < P.nr * D; e += kThreads) {
      const int r = e / D, d = e - (e / D) * D;
      float M = s_m[0][r];
#pragma unroll
      for (int i = 1; i < kWaves; ++i) M = fmaxf(M, s_m[i][r]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        const float f = __builtin_amdgcn_exp2f(s_m[i][r] - M);
        L = fmaf(f, s_l[i][r], L);
        A = fmaf(f, s_acc[i][r][d], A);
      }
      if (ns == 1) {
        const int j = r / P.G, gi = r - (r / P.G) * P.G;
        store_out(op + ((size_t)(b * P.Kq + j) * P.H_q + h * P.G + gi) * D + d, L > 0.f ? A / L : 0.f);
      } else {
        const size_t pr = (bh * P.max_splits + s) * NR + r;
        P.part_acc[pr * D + d] = A;
        if (d == 0) { P.part_ml[2 * pr] = M; P.part_ml[2 * pr + 1] = L; }
      }
    }
    if (ns > 1) {
      __threadfence();
      __syncthreads();
      if (tid == 0) {
        const int old = atomicAdd(&P.counters[bh], 1);
        const int last = (old == ns - 1);
        if (last) atomicExch(&P.counters[bh], 0);
        s_last = last;
      }
      __syncthreads();
      if (s_last) {
        __threadfence();
        for (int e = tid; e < P.nr * D; e += kThreads) {
          const int r = e / D, d = e - (e / D) * D;
          const size_t p0 = (bh * P.max_splits) * NR + r;
          float M = kNegBig;
          for (int i = 0; i < ns; ++i) M = fmaxf(M, P.part_ml[2 * (p0 + (size_t)i * NR)]);
          float L = 0.f, A = 0.f;
          for (int i = 0; i < ns; ++i) {
            const size_t pr = p0 + (size_t)i * NR;
            const float f = __builtin_amdgcn_exp2f(P.part_ml[2 * pr] - M);
            L = fmaf(f, P.part_ml[2 * pr + 1], L);
            A = fmaf(f, P.part_acc[pr * D + d], A);
          }
          const int j = r / P.G, gi = r - (r / P.G) * P.G;
          store_out(op + ((size_t)(b * P.Kq + j) * P.H_q + h * P.G + gi) * D + d, L > 0.f ? A / L : 0.f);
        }
      }
    }
    __syncthreads();  // LDS is reused by the next item
  }
}

template <typename T, int D, int NR>
hipError_t launch_t(const KParams& P, int grid, hipStream_t s) {
  hipLaunchKernelGGL((decode_attention_kernel<T, D, NR>), dim3(grid), dim3(kThreads), 0, s, P);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_nr(const KParams& P, int nr_tmpl, int grid, hipStream_t s) {
  switch (nr_tmpl) {
    case 1: return launch_t<T, D, 1>(P, grid, s);
    case 2: return launch_t<T, D, 2>(P, grid, s);
    case 4: return launch_t<T, D, 4>(P, grid, s);
    case 8: return launch_t<T, D, 8>(P, grid, s);
    case 16: return launch_t<T, D, 16>(P, grid, s);
  }
  return hipErrorInvalidValue;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

bool plan_decode_attention(int B, int Kq, int H_q, int H_kv, int D, int max_kv_len, AttnPlan* p) {
  if (B < 1 || Kq < 1 || H_kv < 1 || H_q % H_kv || max_kv_len < 1) return false;
  const int nr = (H_q / H_kv) * Kq;
  if (nr > 16) return false;
  p->nr = nr;
  p->nr_tmpl = nr <= 1 ? 1 : nr <= 2 ? 2 : nr <= 4 ? 4 : nr <= 8 ? 8 : 16;
  // Aim for ~8192 work items when lengths average half the maximum, in
  // multiples of 64 tokens (16-token tiles x 4 waves), between 64 and 512.
  const double est = (double)B * H_kv * (max_kv_len > 1 ? max_kv_len / 2.0 : 1.0);
  long split = (long)((est / 8192.0 + 63.0) / 64.0) * 64;
  if (split < 64) split = 64;
  if (split > 512) split = 512;
  p->split = (int)split;
  p->max_splits = (int)((max_kv_len + split - 1) / split);
  const size_t slots = (size_t)B * H_kv * p->max_splits * p->nr_tmpl;
  // The counter area has one fixed size, whatever B and H_kv are, so a
  // workspace reused by calls of other shapes never finds partial results
  // where it expects zeroed counters.
  if ((long)B * H_kv > kMaxCounters) return false;
  p->counters_bytes = (size_t)kMaxCounters * sizeof(int);
  p->ml_offset = p->counters_bytes;
  p->acc_offset = p->ml_offset + align256(slots * 2 * sizeof(float));
  p->total_bytes = p->acc_offset + align256(slots * (size_t)D * sizeof(float));
  return true;
}

hipError_t launch_decode_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  KParams P;
  P.q = a.q; P.kc = a.k_cache; P.vc = a.v_cache;
  P.block_table = a.block_table; P.kv_len = a.kv_len; P.o = a.o;
  char* ws = static_cast<char*>(a.workspace);
  P.counters = reinterpret_cast<int*>(ws);
  P.part_ml = reinterpret_cast<float*>(ws + p.ml_offset);
  P.part_acc = reinterpret_cast<float*>(ws + p.acc_offset);
  P.max_blocks = a.max_blocks;
  const long cap = (long)a.max_blocks * a.block_size;
  P.cap = (int)(cap < a.max_kv_len ? cap : a.max_kv_len);
  P.B = a.B; P.Kq = a.Kq; P.H_q = a.H_q; P.H_kv = a.H_kv; P.G = a.H_q / a.H_kv;
  P.nr = p.nr; P.bs = a.block_size; P.num_blocks = a.num_blocks;
  P.split = p.split; P.max_splits = p.max_splits;
  P.scale_log2 = a.scale * kLog2e;
  const long upper = (long)a.B * a.H_kv * p.max_splits;
  const int grid = (int)(upper < 2048 ? upper : 2048);
  if (a.bf16) {
    if (a.D == 128) return launch_nr<uint16_t, 128>(P, p.nr_tmpl, grid, s);
    if (a.D == 64) return launch_nr<uint16_t, 64>(P, p.nr_tmpl, grid, s);
  } else {
    if (a.D == 128) return launch_nr<float, 128>(P, p.nr_tmpl, grid, s);
    if (a.D == 64) return launch_nr<float, 64>(P, p.nr_tmpl, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace clm
