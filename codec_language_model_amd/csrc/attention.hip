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
// query rows that share the KV head are served by one pass over its K/V
// bytes, so every K/V byte is read from HBM once per step.  Each wave owns
// whole items: the grid is persistent, every workgroup derives the item list
// from kv_len (a prefix sum of per-stream split counts, in LDS, built once),
// and its waves stride through the list independently - no barrier, no LDS
// and no cross-workgroup traffic in the main loop.
//
// Inside an item a wave walks 16-token tiles.  The block ids of the item's
// pages are fetched once, one per lane, and picked out with readlane.  Keys
// are read as 16-byte loads, LPR lanes per key row (16 lanes per 256-byte row
// for bf16, D = 128), so one load instruction covers 4 whole rows; the LPR
// partial dot products are summed with DPP inside the 16-lane row.  Values
// are stored transposed inside a block ([D][bs]), so for each of its head
// dimensions a lane reads the run of keys its group scored, contiguous
// across the wave.  The next tile's loads are always in flight while the
// current tile is computed (past the last tile the current one is re-read,
// which hits in cache), so the wait counts stay exact.  Each 16-lane key
// group keeps its own online-softmax state (running max m, sum l,
// accumulator) in registers; the groups merge with shuffles at the end of an
// item.  A stream that fits in one split is written directly; otherwise the
// split's (m, l, acc) goes to the workspace and a second small kernel merges
// the splits of each (stream, KV head) in split order (deterministic).
#include "clm_device.h"
#include "clm_launch.h"

namespace clm {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxB = 4096;

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
  float* part_ml;   // [B][H_kv][max_splits][NR][2]   (m in log2 units, l)
  float* part_acc;  // [B][H_kv][max_splits][NR][D]
  int max_blocks, cap, B, Kq, H_q, H_kv, G, nr, bs, num_blocks, split, max_splits;
  float scale_log2;
};

__device__ __forceinline__ int split_count(int len, const KParams& P) {
  int n = clampi(len, 1, P.cap);
  int s = (n + P.split - 1) / P.split;
  return clampi(s, 1, P.max_splits);
}

template <typename T, int D, int NR, int BS>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(KParams P) {
  using G_ = Geo<T, D>;
  constexpr int LPR = G_::LPR, CPL = G_::CPL, KPG = G_::KPG, DPL = G_::DPL, VE = G_::VE;
  constexpr int NG = G_::NG;
  using VT = typename G_::VT;

  __shared__ int s_prefix[kMaxB + 1];
  __shared__ int s_wsum[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int g = lane / LPR;
  const int c = lane % LPR;
  const int bs = BS ? BS : P.bs;

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
      if (b < P.B) local += split_count(P.kv_len[b], P);
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
        run += split_count(P.kv_len[b], P);
      }
    }
    if (tid == 0) s_prefix[P.B] = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    __syncthreads();
  }
  const int total_items = s_prefix[P.B] * P.H_kv;
  const int nwaves = gridDim.x * kWaves;

  for (int item = blockIdx.x * kWaves + w; item < total_items; item += nwaves) {
    const int u = item / P.H_kv;
    const int h = item - u * P.H_kv;
    int lo = 0, hi = P.B - 1;  // largest b with s_prefix[b] <= u
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (s_prefix[mid] <= u) lo = mid; else hi = mid - 1;
    }
    const int b = uniform(lo);
    const int s = uniform(u - s_prefix[b]);
    const int ns = uniform(s_prefix[b + 1] - s_prefix[b]);

    const int n_total = uniform(clampi(P.kv_len[b], 1, P.cap));
    const int n_min = n_total - (P.Kq - 1);       // keys seen by the first query
    const int t0 = s * P.split;
    const int t1 = min(t0 + P.split, n_total);
    const int n_tiles = (t1 - t0 + 15) >> 4;
    const int p0 = t0 / bs;

    // block ids of the item's pages, one per lane (an item spans <= 64 pages)
    int my_blk = 0;
    {
      const int n_pages = (t1 - 1) / bs - p0 + 1;
      if (lane < n_pages) my_blk = clampi(P.block_table[(size_t)b * P.max_blocks + p0 + lane], 0, P.num_blocks - 1);
    }

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

    auto issue = [&](int ti, uint4 (&kr)[KPG][CPL], VT (&vr)[DPL]) {
      const int tk = t0 + (ti << 4);
      const int blk = __builtin_amdgcn_readlane(my_blk, uniform(tk / bs - p0));
      const int slot0 = tk % bs;
      const size_t hb = (size_t)blk * P.H_kv + h;
      const T* kp = kc + (hb * bs + slot0 + g * KPG) * D + c * VE;
      const T* vp = vc + hb * D * bs + slot0 + (size_t)c * bs + g * KPG;
#pragma unroll
      for (int i = 0; i < KPG; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
          kr[i][cc] = *reinterpret_cast<const uint4*>(kp + i * D + cc * LPR * VE);
#pragma unroll
      for (int jj = 0; jj < DPL; ++jj)
        vr[jj] = *reinterpret_cast<const VT*>(vp + (size_t)jj * LPR * bs);
    };

    // tk: first token of the tile; a tile past the item (tk >= t1) is masked
    // entirely (its loads were a duplicate of the last tile).
    auto compute = [&](int tk, const uint4 (&kr)[KPG][CPL], const VT (&vr)[DPL]) {
      const bool full = tk + 16 <= n_min && tk + 16 <= t1;
      const int vis = tk < t1 ? n_total : 0;   // keys with written slots
      float vf[DPL][KPG];
#pragma unroll
      for (int jj = 0; jj < DPL; ++jj) unpack_v(vr[jj], vf[jj], T());
      if (!full) {
#pragma unroll
        for (int i = 0; i < KPG; ++i) {
          if (tk + g * KPG + i >= vis) {
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
            const int lim = tk < t1 ? n_r[r] : 0;
#pragma unroll
            for (int i = 0; i < KPG; ++i)
              if (tk + g * KPG + i >= lim) sc[i] = -INFINITY;
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
    };

    uint4 ka[KPG][CPL], kb[KPG][CPL];
    VT va[DPL], vb[DPL];
    const int last = n_tiles - 1;
    // Drain the prologue's loads (q, block ids) first, so that at the tile
    // loop's head the only loads in flight are one tile buffer on every path
    // and the waits inside the loop count them exactly.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    issue(0, ka, va);
    // Two tiles per trip, no branch inside: while one buffer is computed the
    // other one's loads are in flight.  Past the last tile, loads re-read the
    // last tile (cache hits) and compute() masks everything.
    for (int ti = 0; ti <= last; ti += 2) {
      issue(min(ti + 1, last), kb, vb);
      compute(t0 + (ti << 4), ka, va);
      issue(min(ti + 2, last), ka, va);
      compute(t0 + ((ti + 1) << 4), kb, vb);
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

    // every lane now holds the merged state for its dims c + LPR*jj; key
    // group g writes the jj in [g*DPL/NG, (g+1)*DPL/NG) (all jj if DPL < NG)
    constexpr int JPG = DPL >= NG ? DPL / NG : DPL;
    const int jbase = DPL >= NG ? g * JPG : 0;
    const bool writer = DPL >= NG ? true : (g == 0);
    const size_t bh = (size_t)b * P.H_kv + h;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (r < P.nr && writer) {
        if (ns == 1) {
          const int j = r / P.G, gi = r - (r / P.G) * P.G;
          T* orow = op + ((size_t)(b * P.Kq + j) * P.H_q + h * P.G + gi) * D;
          const float inv = l[r] > 0.f ? 1.f / l[r] : 0.f;
#pragma unroll
          for (int k = 0; k < JPG; ++k) {
            const int jj = jbase + k;
            store_out(orow + c + LPR * jj, acc[r][jj] * inv);
          }
        } else {
          const size_t pr = (bh * P.max_splits + s) * NR + r;
#pragma unroll
          for (int k = 0; k < JPG; ++k) {
            const int jj = jbase + k;
            P.part_acc[pr * D + c + LPR * jj] = acc[r][jj];
          }
          if (lane == 0) { P.part_ml[2 * pr] = m[r]; P.part_ml[2 * pr + 1] = l[r]; }
        }
      }
    }
  }
}

// Merge the splits of each (stream, KV head) that has more than one, in split
// order: o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
template <typename T, int D, int NR>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(KParams P) {
  const int bh = blockIdx.x;
  const int b = bh / P.H_kv;
  const int h = bh - b * P.H_kv;
  const int ns = split_count(P.kv_len[b], P);
  if (ns <= 1) return;
  T* __restrict__ op = static_cast<T*>(P.o);
  for (int e = threadIdx.x; e < P.nr * D; e += kThreads) {
    const int r = e / D, d = e - (e / D) * D;
    const size_t p0 = (size_t)bh * P.max_splits * NR + r;
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

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <typename T, int D, int NR>
hipError_t launch_t(const KParams& P, int grid, hipStream_t s) {
  if (P.bs == 16)
    hipLaunchKernelGGL((attn_split_kernel<T, D, NR, 16>), dim3(grid), dim3(kThreads), 0, s, P);
  else
    hipLaunchKernelGGL((attn_split_kernel<T, D, NR, 0>), dim3(grid), dim3(kThreads), 0, s, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P.max_splits <= 1) return e;
  hipLaunchKernelGGL((attn_combine_kernel<T, D, NR>), dim3(P.B * P.H_kv), dim3(kThreads), 0, s, P);
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
  // Aim for ~16k wave work items when lengths average half the maximum; a
  // split is a multiple of 64 tokens between 64 and 256 (an item then spans
  // at most 17 blocks of 16 tokens).
  const double est = (double)B * H_kv * (max_kv_len > 1 ? max_kv_len / 2.0 : 1.0);
  long split = (long)((est / 16384.0 + 63.0) / 64.0) * 64;
  if (split < 64) split = 64;
  if (split > 256) split = 256;
  p->split = (int)split;
  p->max_splits = (int)((max_kv_len + split - 1) / split);
  const size_t slots = (size_t)B * H_kv * p->max_splits * p->nr_tmpl;
  p->ml_offset = 0;
  p->acc_offset = align256(slots * 2 * sizeof(float));
  p->total_bytes = p->acc_offset + align256(slots * (size_t)D * sizeof(float));
  return true;
}

hipError_t launch_decode_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  KParams P;
  P.q = a.q; P.kc = a.k_cache; P.vc = a.v_cache;
  P.block_table = a.block_table; P.kv_len = a.kv_len; P.o = a.o;
  char* ws = static_cast<char*>(a.workspace);
  P.part_ml = reinterpret_cast<float*>(ws + p.ml_offset);
  P.part_acc = reinterpret_cast<float*>(ws + p.acc_offset);
  P.max_blocks = a.max_blocks;
  const long cap = (long)a.max_blocks * a.block_size;
  P.cap = (int)(cap < a.max_kv_len ? cap : a.max_kv_len);
  P.B = a.B; P.Kq = a.Kq; P.H_q = a.H_q; P.H_kv = a.H_kv; P.G = a.H_q / a.H_kv;
  P.nr = p.nr; P.bs = a.block_size; P.num_blocks = a.num_blocks;
  P.split = p.split; P.max_splits = p.max_splits;
  P.scale_log2 = a.scale * kLog2e;
  const long items = (long)a.B * a.H_kv * p.max_splits;       // upper bound
  const long want = (items + kWaves - 1) / kWaves;
  const long cap_wg = 3L * device_cus();
  const int grid = (int)(want < cap_wg ? want : cap_wg);
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
