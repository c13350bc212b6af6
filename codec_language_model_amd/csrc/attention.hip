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
// bytes, so every K/V byte is read from HBM once per step.  The grid is
// persistent: every workgroup rebuilds the item numbering from kv_len once
// (stream lengths and prefix sums in LDS) - first every full-size split of
// every stream, then each stream's shorter last split, longest first - and
// its waves take items in a snake order over the grid's waves.  (A shared
// ticket counter balanced the tail better but cost more: device-wide atomics
// on one address serialise across the chip.)  While a wave streams one item
// it already loads the next item's block ids and query slice.  No barrier or
// cross-wave traffic in the main loop.
//
// Inside an item a wave walks 16-token tiles.  The block ids of the item's
// pages are fetched once, one per lane, and picked out with readlane.  Keys
// are read as 16-byte loads, LPR lanes per key row (16 lanes per 256-byte row
// for bf16, D = 128), so one load instruction covers 4 whole rows; the LPR
// partial dot products are summed with DPP inside the 16-lane row.  K and V
// are read with non-temporal loads: every byte is used once per call, and on
// gfx950 that policy streams scattered 4 KiB pages faster than the default.
// Values are stored transposed inside a block ([D][bs]), so for each of its
// head dimensions a lane reads the run of keys its group scored, contiguous
// across the wave.  The loop body covers two tiles without a branch: while
// one tile buffer is computed the other's loads are in flight (past the last
// tile the loads read one shared tile that stays in L2, and the tile is
// masked), so the wait counts stay exact.  Each 16-lane key group keeps its
// own online-softmax state (running max m, sum l, accumulator) in registers;
// the groups merge with shuffles at the end of an item.  A stream that fits
// in one split is written directly; otherwise the split's (m, l, acc) goes to
// the workspace and a second kernel merges the splits of each row in split
// order.
//
// Blocks of 3..16 query rows per KV head, and every FP8 cache, use the
// matrix-core kernel (attn_mfma_kernel): S = K.q^T and O^T += V^T.P^T per tile
// on the MFMA units.  Up to kRingMaxB streams, its tiles reach LDS by
// global-to-LDS DMA into a per-wave ring of kRingStages stages, so three tiles
// are in flight per wave without holding registers.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "clm_device.h"
#include "clm_launch.h"

// Split partials of clm_decode_attention_noalloc: the library's own scratch,
// one copy per GPU for the life of the process (zero-filled at load; the
// attention kernels need no initial contents).  Host code never passes this
// name to a kernel: it is a host-side stand-in, so the device address comes
// from hipGetSymbolAddress, once per device (clm::attention_scratch).
static __device__ __align__(256) uint8_t scratch[clm::kAttentionScratchBytes];

namespace clm {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxB = 4096;
constexpr int kRingMaxB = 512;       // streams the LDS-staged matrix-core kernel takes
constexpr int kRingStages = 4;       // its per-wave ring of tile stages

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
__device__ __forceinline__ void to_words(uint32_t v, uint32_t* w) { w[0] = v; }
__device__ __forceinline__ void to_words(uint2 v, uint32_t* w) { w[0] = v.x; w[1] = v.y; }
__device__ __forceinline__ void to_words(uint4 v, uint32_t* w) { w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w; }

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
  const float* k_scale;   // FP8 cache: [num_blocks][H_kv][bs] per-row scales
  const float* v_scale;
  float* part_ml;   // [B][H_kv][max_splits][NR][2]   (m in log2 units, l)
  float* part_acc;  // [B][H_kv][max_splits][NR][D]
  int max_blocks, cap, B, Kq, H_q, H_kv, G, nr, bs, num_blocks, split, max_splits;
  float scale_log2;
};

// Values are stored [D][bs] inside a block, so a 16-token tile reads 16 of a
// head dimension's bs slots.  With 16-slot pages that is the whole row and
// the load streams (non-temporal); with longer pages the rest of each line
// belongs to the item's next tiles, so it is loaded with the default policy
// and stays in L2 for them.
template <int BS, class V>
__device__ __forceinline__ V ld_values(const V* p) {
  if constexpr (BS == 16) return ld_nt(p);
  else return *p;
}

__device__ __forceinline__ int stream_len(int len, const KParams& P) { return clampi(len, 1, P.cap); }
__device__ __forceinline__ int full_splits(int n, const KParams& P) { return min(n / P.split, P.max_splits); }
__device__ __forceinline__ int split_count(int n, const KParams& P) {
  return clampi((n + P.split - 1) / P.split, 1, P.max_splits);
}

// Exclusive block-wide prefix over B per-stream counts, into s[0..B].
template <class F>
__device__ void block_prefix(int* s, int* s_wsum, int B, F count) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (B + kThreads - 1) / kThreads;
  const int b0 = tid * per;
  int local = 0;
  for (int k = 0; k < per; ++k)
    if (b0 + k < B) local += count(b0 + k);
  const int incl = wave_incl_scan_i(local);
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  int run = incl - local;
  for (int i = 0; i < w; ++i) run += s_wsum[i];
  for (int k = 0; k < per; ++k) {
    if (b0 + k < B) {
      s[b0 + k] = run;
      run += count(b0 + k);
    }
  }
  if (tid == 0) s[B] = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
  __syncthreads();
}

// largest b in [0, B) with s[b] <= u (s non-decreasing, s[0] = 0)
__device__ __forceinline__ int find_stream(const int* s, int B, int u) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The streams whose last split is shorter than `split`, ordered by that
// split's length bin (1..16, 16 = longest) descending, then by stream index:
// s[0..n).  A counting sort (ballots per bin up to one stream per thread,
// else one block-wide scan per bin), so every workgroup builds the same list.
// bin(b) = 0 means no short split.  Returns n.
template <class F>
__device__ int short_splits_sorted(int* s, int (*s_bins)[16], int B, F bin) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (B <= kThreads) {
    // one stream per thread: per bin, one ballot gives the wave's count and
    // each lane's rank among the wave's lanes in that bin (lanes in stream
    // order), so the list comes out of one barrier and no scans
    const int t = tid < B ? bin(tid) : 0;
    const uint64_t below = (uint64_t(1) << lane) - 1;
    int rank = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(t == 16 - k);
      if (lane == 0) s_bins[w][k] = __popcll(m);
      if (t == 16 - k) rank = __popcll(m & below);
    }
    __syncthreads();
    int total = 0, pos = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      int tot = 0, before = 0;
      for (int i = 0; i < kWaves; ++i) {
        const int c = s_bins[i][k];
        before += i < w ? c : 0;
        tot += c;
      }
      if (t == 16 - k) pos = total + before + rank;
      total += tot;
    }
    if (t > 0) s[pos] = tid;
    __syncthreads();
    return total;
  }
  const int per = (B + kThreads - 1) / kThreads;
  const int b0 = tid * per;
  int cnt[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) cnt[k] = 0;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    const int t = b < B ? bin(b) : 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) cnt[k] += (t == 16 - k);
  }
  int excl[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int incl = wave_incl_scan_i(cnt[k]);
    excl[k] = incl - cnt[k];
    if (lane == 63) s_bins[w][k] = incl;
  }
  __syncthreads();
  int start = 0, n = 0;
  int pos[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    int before = 0, tot = 0;
    for (int i = 0; i < kWaves; ++i) {
      before += i < w ? s_bins[i][k] : 0;
      tot += s_bins[i][k];
    }
    pos[k] = start + before + excl[k];
    start += tot;
  }
  n = start;
  for (int i = 0; i < per; ++i) {
    const int b = b0 + i;
    const int t = b < B ? bin(b) : 0;
    if (t > 0) {
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (t == 16 - k) s[pos[k]++] = b;
    }
  }
  __syncthreads();
  return n;
}

template <typename T, int D, int NR, int BS, bool EXACT>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(KParams P) {
  using G_ = Geo<T, D>;
  constexpr int LPR = G_::LPR, CPL = G_::CPL, KPG = G_::KPG, DPL = G_::DPL, VE = G_::VE;
  constexpr int NG = G_::NG;
  using VT = typename G_::VT;

  __shared__ int s_full[kMaxB + 1];   // prefix of full-size splits per stream
  __shared__ int s_plist[kMaxB];      // streams with a short last split, longest first
  __shared__ int s_bins[kWaves][16];
  __shared__ int s_len[kMaxB];        // clamped stream lengths
  __shared__ int s_wsum[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int g = lane / LPR;
  const int c = lane % LPR;
  const int bs = BS ? BS : P.bs;
  // query rows of this call: NR exactly when EXACT (no per-row test)
  const int nrow = EXACT ? NR : P.nr;

  const T* __restrict__ qp = static_cast<const T*>(P.q);
  const T* __restrict__ kc = static_cast<const T*>(P.kc);
  const T* __restrict__ vc = static_cast<const T*>(P.vc);
  T* __restrict__ op = static_cast<T*>(P.o);

  for (int b = tid; b < P.B; b += kThreads) s_len[b] = stream_len(P.kv_len[b], P);
  __syncthreads();
  block_prefix(s_full, s_wsum, P.B, [&](int b) { return full_splits(s_len[b], P); });
  // short last splits, binned by length in sixteenths of a split
  const int tps = P.split >> 4;
  const int n_part = short_splits_sorted(s_plist, s_bins, P.B, [&](int b) {
    const int rem = s_len[b] - full_splits(s_len[b], P) * P.split;
    return rem > 0 ? (((rem + 15) >> 4) * 16 + tps - 1) / tps : 0;
  });
  const int n_full = s_full[P.B] * P.H_kv;
  const int total_items = n_full + n_part * P.H_kv;
  const int nw_total = gridDim.x * kWaves;

  // item -> (stream, split, KV head), from LDS only
  auto locate = [&](int item, int& b, int& s, int& h) {
    if (item < n_full) {
      const int u = item / P.H_kv;
      h = item - u * P.H_kv;
      b = find_stream(s_full, P.B, u);
      s = u - s_full[b];
    } else {
      const int t = item - n_full;
      const int u = t / P.H_kv;
      h = t - u * P.H_kv;
      b = s_plist[u];
      s = s_full[b + 1] - s_full[b];   // the last split follows the full ones
    }
    b = uniform(b);
    s = uniform(s);
    h = uniform(h);
  };
  // the item's block ids (one page per lane; an item spans <= 64 pages) and
  // this lane's slice of its query rows
  auto fetch = [&](int item, int& blk, uint32_t (&qv)[NR][4 * CPL]) {
    int b, s, h;
    locate(item, b, s, h);
    const int n = s_len[b];
    const int t0 = s * P.split;
    const int t1 = min(t0 + P.split, n);
    const int p0 = t0 / bs;
    const int n_pages = (t1 - 1) / bs - p0 + 1;
    blk = 0;
    if (lane < n_pages) blk = clampi(P.block_table[(size_t)b * P.max_blocks + p0 + lane], 0, P.num_blocks - 1);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int i = 0; i < 4 * CPL; ++i) qv[r][i] = 0u;
      if (r < nrow) {
        const int j = r / P.G, gi = r - (r / P.G) * P.G;
        const T* qrow = qp + ((size_t)(b * P.Kq + j) * P.H_q + h * P.G + gi) * D;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) {
          const uint4 v = *reinterpret_cast<const uint4*>(qrow + (c + cc * LPR) * VE);
          qv[r][cc * 4 + 0] = v.x; qv[r][cc * 4 + 1] = v.y;
          qv[r][cc * 4 + 2] = v.z; qv[r][cc * 4 + 3] = v.w;
        }
      }
    }
  };

  // The next item's block ids and query slice are loaded while this one
  // streams.  Snake deal: round r gives wave w item r*nw + (r even ? w : nw-1-w).  The
  // items are ordered longest first, so the waves that took the longest
  // items of one round take the shortest of the next.
  const int my_w = blockIdx.x * kWaves + (tid >> 6);
  int round_ = 0;
  auto deal = [&](int r) { return r * nw_total + ((r & 1) ? nw_total - 1 - my_w : my_w); };
  int item = deal(0);
  int my_blk = 0;
  uint32_t qw[NR][4 * CPL];
  if (item < total_items) fetch(item, my_blk, qw);

  while (item < total_items) {
    const int next_item = deal(++round_);
    int b, s, h;
    locate(item, b, s, h);
    const int n_total = s_len[b];
    const int ns = split_count(n_total, P);
    const int n_min = n_total - (P.Kq - 1);       // keys seen by the first query
    const int t0 = s * P.split;
    const int t1 = min(t0 + P.split, n_total);
    const int n_tiles = (t1 - t0 + 15) >> 4;
    const int p0 = t0 / bs;
    int n_r[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) n_r[r] = r < nrow ? n_total - (P.Kq - 1 - r / P.G) : 0;

    float m[NR], l[NR], acc[NR][DPL];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      m[r] = kNegBig;
      l[r] = 0.f;
#pragma unroll
      for (int jj = 0; jj < DPL; ++jj) acc[r][jj] = 0.f;
    }

    // A tile past the item's end (the pipeline's tail) reads slots 0..15 of
    // block 0, KV head 0 instead: the same bytes for every wave, so they stay
    // in L2 rather than costing HBM reads.  Such a tile is masked entirely.
    auto issue = [&](int ti, uint4 (&kr)[KPG][CPL], VT (&vr)[DPL]) {
      const bool past = ti >= n_tiles;
      const int tk = t0 + (ti << 4);
      const int blk = past ? 0 : __builtin_amdgcn_readlane(my_blk, uniform(min(tk / bs - p0, 63)));
      const int slot0 = past ? 0 : tk % bs;
      const size_t hb = past ? 0 : (size_t)blk * P.H_kv + h;
      const T* kp = kc + (hb * bs + slot0 + g * KPG) * D + c * VE;
      const T* vp = vc + hb * D * bs + slot0 + (size_t)c * bs + g * KPG;
#pragma unroll
      for (int i = 0; i < KPG; ++i)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc)
          kr[i][cc] = ld_nt(reinterpret_cast<const uint4*>(kp + i * D + cc * LPR * VE));
#pragma unroll
      for (int jj = 0; jj < DPL; ++jj)
        vr[jj] = ld_values<BS>(reinterpret_cast<const VT*>(vp + (size_t)jj * LPR * bs));
    };

    // P.V for one tile; MASK zeroes value lanes of keys past `vis` (slots
    // that may hold anything, NaN included).  bf16: the transposed block
    // layout puts a head dimension's values for two consecutive keys in one
    // 32-bit word, so the products go through v_dot2_f32_bf16 against the
    // probabilities packed to bf16 pairs (fp32 accumulation); fp32: FMAs.
    auto pv = [&](auto mask_tag, const VT (&vr)[DPL], const float (&p)[NR][KPG], const float (&corr)[NR],
                  int tk, int vis) {
      constexpr bool MASK = decltype(mask_tag)::value;
      if constexpr (std::is_same<T, uint16_t>::value) {
        constexpr int NW = KPG / 2;
        uint32_t pk[NR][NW];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int i2 = 0; i2 < NW; ++i2) pk[r][i2] = pack_bf16x2(p[r][2 * i2], p[r][2 * i2 + 1]);
        uint32_t keep[NW];
#pragma unroll
        for (int i2 = 0; i2 < NW; ++i2) {
          const int t = tk + g * KPG + 2 * i2;
          keep[i2] = (t < vis ? 0x0000ffffu : 0u) | (t + 1 < vis ? 0xffff0000u : 0u);
        }
#pragma unroll
        for (int jj = 0; jj < DPL; ++jj) {
          uint32_t wv[NW];
          to_words(vr[jj], wv);
          if (MASK) {
#pragma unroll
            for (int i2 = 0; i2 < NW; ++i2) wv[i2] &= keep[i2];
          }
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (r < nrow) {
              float a = acc[r][jj] * corr[r];
#pragma unroll
              for (int i2 = 0; i2 < NW; ++i2) a = dot2_bf16(pk[r][i2], wv[i2], a);
              acc[r][jj] = a;
            }
          }
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < DPL; ++jj) {
          float vf[KPG];
          unpack_v(vr[jj], vf, T());
          if (MASK) {
#pragma unroll
            for (int i = 0; i < KPG; ++i) vf[i] = (tk + g * KPG + i < vis) ? vf[i] : 0.f;
          }
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (r < nrow) {
              float a = acc[r][jj] * corr[r];
#pragma unroll
              for (int i = 0; i < KPG; ++i) a = fmaf(p[r][i], vf[i], a);
              acc[r][jj] = a;
            }
          }
        }
      }
    };

    // tk: first token of the tile; a tile past the item (tk >= t1) is masked
    // entirely (its loads read the shared block-0 tile).  No branch:
    // the key masks are applied on every tile (all-pass on full tiles), which
    // costs a few selects but keeps the accumulators in place.
    auto compute = [&](int tk, const uint4 (&kr)[KPG][CPL], const VT (&vr)[DPL]) {
      const int vis = tk < t1 ? n_total : 0;   // keys whose slots are written
      float p[NR][KPG], corr[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        corr[r] = 1.f;
#pragma unroll
        for (int i = 0; i < KPG; ++i) p[r][i] = 0.f;
        if (r < nrow) {
          const int lim = tk < t1 ? n_r[r] : 0;
          float sc[KPG];
#pragma unroll
          for (int i = 0; i < KPG; ++i) {
            float part = 0.f;
#pragma unroll
            for (int cc = 0; cc < CPL; ++cc) part = chunk_dot(&qw[r][cc * 4], kr[i][cc], part, T());
            const float sum = group_sum<LPR>(part) * P.scale_log2;   // every lane of the row
            sc[i] = tk + g * KPG + i < lim ? sum : -INFINITY;
          }
          float mx = sc[0];
#pragma unroll
          for (int i = 1; i < KPG; ++i) mx = fmaxf(mx, sc[i]);
          const float m_new = fmaxf(m[r], mx);
          corr[r] = __builtin_amdgcn_exp2f(m[r] - m_new);
          float psum = 0.f;
#pragma unroll
          for (int i = 0; i < KPG; ++i) {
            p[r][i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
            psum += p[r][i];
          }
          l[r] = l[r] * corr[r] + psum;
          m[r] = m_new;
        }
      }
      pv(std::true_type(), vr, p, corr, tk, vis);
    };

    uint4 ka[KPG][CPL], kb[KPG][CPL];
    VT va[DPL], vb[DPL];
    const int last = n_tiles - 1;
    // Drain what is still in flight (the previous item's trailing tile past
    // its end, an L2 hit) so that the tile loop's waits count exactly.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    issue(0, ka, va);
    int nblk = 0;
    uint32_t nq[NR][4 * CPL];
    if (next_item < total_items) fetch(next_item, nblk, nq);
    for (int ti = 0; ti <= last; ti += 2) {
      issue(ti + 1, kb, vb);
      compute(t0 + (ti << 4), ka, va);
      issue(ti + 2, ka, va);
      compute(t0 + ((ti + 1) << 4), kb, vb);
    }

    // ---- merge the key groups of this wave (lanes c, c+LPR, c+2LPR, ...) -----
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (r < nrow) {
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
      if (r < nrow && writer) {
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
    item = next_item;
    my_blk = nblk;
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int i = 0; i < 4 * CPL; ++i) qw[r][i] = nq[r][i];
  }
}

// Matrix-core variant for bf16 blocks of up to 16 query rows per KV head (a
// verification block of K drafted positions times the GQA group).  Same work
// items and item order as attn_split_kernel; per 16-token tile:
//   S[t][r]  = sum_d K[t][d] q[r][d]      four (D/32) v_mfma_f32_16x16x32_bf16,
//              A = K (16 tokens x 32 dims), B = q (32 dims x 16 rows)
//   online softmax per row r on S; lane l holds tokens 4*(l/16)..+3 of row
//   l%16, so a row's max needs two cross-lane steps and its sum none (lanes
//   keep partial sums, added at the end of the item)
//   O^T[e][r] += sum_t V[t][e] P[r][t]    eight (D/16) v_mfma_f32_16x16x16_bf16,
//              A = V^T (16 dims x 16 tokens: the transposed value block gives
//              each lane 4 consecutive tokens of one dim, one 8-byte load),
//              B = P^T (16 tokens x 16 rows: exactly the layout S came out in)
// Per lane: 4 score, D/2 accumulator and D/8 query registers, whatever the
// row count, where the vector kernel needs NR*D/16 accumulators per lane.
// Four E4M3 bytes -> four bf16 values in two words (exact: every E4M3 value
// is a bf16 value), with gfx950's scaled fp8 -> bf16 pair conversion at
// scale 1: one instruction per two values.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

template <int D, int NR, int BS, bool F8, bool RING = false>
__global__ __launch_bounds__(kThreads, 2) void attn_mfma_kernel(KParams P) {
  typedef short bf16x4s __attribute__((ext_vector_type(4)));
  // K/V element: bf16, or E4M3 bytes with one fp32 scale per (token, KV head)
  using KT = typename std::conditional<F8, uint2, bf16x8_t>::type;    // 8 keys-dims per lane
  using VTy = typename std::conditional<F8, uint32_t, uint2>::type;   // 4 tokens per lane
  using E = typename std::conditional<F8, uint8_t, uint16_t>::type;
  constexpr int NS = D / 32;   // score MFMAs per tile
  constexpr int NJ = D / 16;   // value MFMAs per tile
  static_assert(NR <= 16, "one MFMA column block of query rows");
  // LDS ring: per wave kRingStages stages of one tile each.  FP8: keys
  // [D/8 groups][16 slots][8 B], values [D dims][16 slots], then the 16 key
  // scales and 16 value scales (and a copy of both).  bf16: keys [16 slots][D]
  // with the 16-byte chunks of slot r XOR-swizzled by r (bank-conflict-free
  // operand reads), values [D dims][16 slots].
  constexpr int kStageB = F8 ? 32 * D + 256 : 64 * D;
  constexpr int MB = RING ? kRingMaxB : kMaxB;

  __shared__ int s_full[MB + 1];
  __shared__ int s_plist[MB];
  __shared__ int s_bins[kWaves][16];
  __shared__ int s_len[MB];
  __shared__ int s_wsum[kWaves];
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[RING ? kWaves * kRingStages * kStageB : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int bs = BS ? BS : P.bs;
  const int nrow = P.nr;

  const uint16_t* __restrict__ qp = static_cast<const uint16_t*>(P.q);
  const E* __restrict__ kc = static_cast<const E*>(P.kc);
  const E* __restrict__ vc = static_cast<const E*>(P.vc);
  uint16_t* __restrict__ op = static_cast<uint16_t*>(P.o);

  for (int b = tid; b < P.B; b += kThreads) s_len[b] = stream_len(P.kv_len[b], P);
  __syncthreads();
  block_prefix(s_full, s_wsum, P.B, [&](int b) { return full_splits(s_len[b], P); });
  const int tps = P.split >> 4;
  const int n_part = short_splits_sorted(s_plist, s_bins, P.B, [&](int b) {
    const int rem = s_len[b] - full_splits(s_len[b], P) * P.split;
    return rem > 0 ? (((rem + 15) >> 4) * 16 + tps - 1) / tps : 0;
  });
  const int n_full = s_full[P.B] * P.H_kv;
  const int total_items = n_full + n_part * P.H_kv;
  const int nw_total = gridDim.x * kWaves;

  auto locate = [&](int item, int& b, int& s, int& h) {
    if (item < n_full) {
      const int u = item / P.H_kv;
      h = item - u * P.H_kv;
      b = find_stream(s_full, P.B, u);
      s = u - s_full[b];
    } else {
      const int t = item - n_full;
      const int u = t / P.H_kv;
      h = t - u * P.H_kv;
      b = s_plist[u];
      s = s_full[b + 1] - s_full[b];
    }
    b = uniform(b);
    s = uniform(s);
    h = uniform(h);
  };
  // block ids (one page per lane) and this lane's query fragments: row l%16,
  // dims 32*k + 8*(l/16) .. +7 for k < NS (zeros for rows past the block)
  auto fetch = [&](int item, int& blk, bf16x8_t (&qf)[NS]) {
    int b, s, h;
    locate(item, b, s, h);
    const int n = s_len[b];
    const int t0 = s * P.split;
    const int t1 = min(t0 + P.split, n);
    const int p0 = t0 / bs;
    const int n_pages = (t1 - 1) / bs - p0 + 1;
    blk = 0;
    if (lane < n_pages) blk = clampi(P.block_table[(size_t)b * P.max_blocks + p0 + lane], 0, P.num_blocks - 1);
#pragma unroll
    for (int k = 0; k < NS; ++k) qf[k] = bf16x8_t{};
    if (l16 < nrow) {
      const int j = l16 / P.G, gi = l16 - (l16 / P.G) * P.G;
      const uint16_t* qrow = qp + ((size_t)(b * P.Kq + j) * P.H_q + h * P.G + gi) * D + 8 * lg;
#pragma unroll
      for (int k = 0; k < NS; ++k) qf[k] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * k);
    }
  };

  // Snake deal: round r gives wave w item r*nw + (r even ? w : nw-1-w).  The
  // items are ordered longest first, so the waves that took the longest
  // items of one round take the shortest of the next.
  const int my_w = blockIdx.x * kWaves + (tid >> 6);
  int round_ = 0;
  auto deal = [&](int r) { return r * nw_total + ((r & 1) ? nw_total - 1 - my_w : my_w); };
  int item = deal(0);
  int my_blk = 0;
  bf16x8_t qf[NS];
  if (item < total_items) fetch(item, my_blk, qf);

  while (item < total_items) {
    const int next_item = deal(++round_);
    int b, s, h;
    locate(item, b, s, h);
    const int n_total = s_len[b];
    const int ns = split_count(n_total, P);
    const int t0 = s * P.split;
    const int t1 = min(t0 + P.split, n_total);
    const int n_tiles = (t1 - t0 + 15) >> 4;
    const int p0 = t0 / bs;
    // keys visible to this lane's query row (0 for rows past the block)
    const int n_row = l16 < nrow ? n_total - (P.Kq - 1 - l16 / P.G) : 0;

    float m = kNegBig, lsum = 0.f;
    f32x4_t acc[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // a tile past the item's end reads block 0, KV head 0 (kept in L2; the
    // tile is masked entirely), as in attn_split_kernel
    auto issue = [&](int ti, KT (&kr)[NS], VTy (&vr)[NJ], float4& ks, float4& vs) {
      const bool past = ti >= n_tiles;
      const int tk = t0 + (ti << 4);
      const int blk = past ? 0 : __builtin_amdgcn_readlane(my_blk, uniform(min(tk / bs - p0, 63)));
      const int slot0 = past ? 0 : tk % bs;
      const size_t hb = past ? 0 : (size_t)blk * P.H_kv + h;
      const E* kp = kc + (hb * bs + slot0 + l16) * D + 8 * lg;
      const E* vp = vc + hb * D * bs + (size_t)l16 * bs + slot0 + 4 * lg;
      if constexpr (F8) {
        // keys in 8-dimension groups [block][head][d/8][slot][8]: lane (token
        // l%16, group 4k + l/16) reads 8 bytes, and one instruction reads 4
        // whole groups of the tile's 16 keys (512 contiguous bytes at bs 16)
        const E* kg = kc + ((hb * (D / 8) + lg) * bs + slot0 + l16) * 8;
#pragma unroll
        for (int k = 0; k < NS; ++k) kr[k] = ld_nt(reinterpret_cast<const uint2*>(kg + (size_t)32 * k * bs));
#pragma unroll
        for (int j = 0; j < NJ; ++j) vr[j] = ld_values<BS>(reinterpret_cast<const uint32_t*>(vp + (size_t)16 * j * bs));
        ks = *reinterpret_cast<const float4*>(P.k_scale + hb * bs + slot0 + 4 * lg);
        vs = *reinterpret_cast<const float4*>(P.v_scale + hb * bs + slot0 + 4 * lg);
      } else {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          const uint4 w = ld_nt(reinterpret_cast<const uint4*>(kp + 32 * k));
          kr[k] = __builtin_bit_cast(bf16x8_t, w);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) vr[j] = ld_values<BS>(reinterpret_cast<const uint2*>(vp + (size_t)16 * j * bs));
      }
    };

    // tk: first token of the tile; tiles past the item (tk >= t1) are
    // masked entirely
    auto compute = [&](int tk, const KT (&kr)[NS], const VTy (&vr)[NJ], const float4& ks, const float4& vs) {
      f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        bf16x8_t a;
        if constexpr (F8) {
          const uint2 lo = fp8x4_to_bf16x4(kr[k].x), hi = fp8x4_to_bf16x4(kr[k].y);
          a = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        } else {
          a = kr[k];
        }
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[k], S, 0, 0, 0);
      }
      const int lim = tk < t1 ? n_row : 0;
      const int tl = tk + 4 * lg;                 // this lane's first token
      float kscale[4] = {1.f, 1.f, 1.f, 1.f};
      if constexpr (F8) { kscale[0] = ks.x; kscale[1] = ks.y; kscale[2] = ks.z; kscale[3] = ks.w; }
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] = tl + i < lim ? S[i] * kscale[i] * P.scale_log2 : -INFINITY;
      float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m, mx);
      const float corr = __builtin_amdgcn_exp2f(m - m_new);
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
      lsum = lsum * corr + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      m = m_new;
      // values of slots that hold no key yet may be anything (NaN): zero them
      const int vis = tk < t1 ? n_total : 0;
      float pv[4] = {pr[0], pr[1], pr[2], pr[3]};
      if constexpr (F8) {                         // the value scale folds into P
        const float vsc[4] = {vs.x, vs.y, vs.z, vs.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = tl + i < vis ? pr[i] * vsc[i] : 0.f;
      }
      const uint32_t p01 = pack_bf16x2(pv[0], pv[1]), p23 = pack_bf16x2(pv[2], pv[3]);
      const bf16x4s pb = __builtin_bit_cast(bf16x4s, make_uint2(p01, p23));
      // rescale the accumulators only when some row's maximum rose in this
      // tile (corr is exactly 1 otherwise): after the first tiles of an item
      // most tiles skip it
      if (__builtin_amdgcn_ballot_w64(corr != 1.f)) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[j] = acc[j] * corr;
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        uint2 vw;
        if constexpr (F8) {
          const uint32_t keep = (tl < vis ? 0xffu : 0u) | (tl + 1 < vis ? 0xff00u : 0u) |
                                (tl + 2 < vis ? 0xff0000u : 0u) | (tl + 3 < vis ? 0xff000000u : 0u);
          vw = fp8x4_to_bf16x4(vr[j] & keep);
        } else {
          const uint32_t keep0 = (tl < vis ? 0x0000ffffu : 0u) | (tl + 1 < vis ? 0xffff0000u : 0u);
          const uint32_t keep1 = (tl + 2 < vis ? 0x0000ffffu : 0u) | (tl + 3 < vis ? 0xffff0000u : 0u);
          vw = make_uint2(vr[j].x & keep0, vr[j].y & keep1);
        }
        const bf16x4s va = __builtin_bit_cast(bf16x4s, vw);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, acc[j], 0, 0, 0);
      }
    };

    int nblk = 0;
    bf16x8_t nq[NS];
    if constexpr (RING) {
      // Tiles reach LDS by DMA into this wave's ring (no registers held while
      // in flight, no barrier: only this wave touches its stages).  Tile ti
      // lives in stage ti % kRingStages; kRingStages - 1 tiles are in flight
      // while one is multiplied.
      constexpr int kOps = F8 ? D / 32 + 1 : D / 16;   // DMA instructions per tile
      constexpr int kCh = D / 8;                        // bf16: 16-byte chunks per key row
      uint8_t* ring = s_ring + (tid >> 6) * (kRingStages * kStageB);
      const uint32_t ring_lds = (uint32_t)reinterpret_cast<uintptr_t>(ring);
      const uint8_t* __restrict__ kc8 = reinterpret_cast<const uint8_t*>(P.kc);
      const uint8_t* __restrict__ vc8 = reinterpret_cast<const uint8_t*>(P.vc);
      auto dma_tile = [&](int ti) {
        const bool past = ti >= n_tiles;   // past the item: block 0, KV head 0 (L2)
        const int tk = t0 + (ti << 4);
        const int blk = past ? 0 : __builtin_amdgcn_readlane(my_blk, uniform(min(tk / bs - p0, 63)));
        const int slot0 = past ? 0 : tk % bs;
        const size_t hb = past ? 0 : (size_t)blk * P.H_kv + h;
        const uint32_t base = ring_lds + (uint32_t)((ti & (kRingStages - 1)) * kStageB);
        if constexpr (F8) {
          // keys: instruction i, lane l: group 8 i + l/8, bytes 16 (l%8) of its 128
#pragma unroll
          for (int i = 0; i < D / 64; ++i)
            dma16(kc8 + ((hb * (D / 8) + 8 * i + (lane >> 3)) * bs + slot0) * 8 + 16 * (lane & 7),
                  uniform(base + 1024 * i));
          // values: instruction i, lane l: dimension 64 i + l, its 16 slots
#pragma unroll
          for (int i = 0; i < D / 64; ++i)
            dma16(vc8 + (hb * D + 64 * i + lane) * bs + slot0, uniform(base + 16 * D + 1024 * i));
          // scales: lanes 0-15 key scales, 16-31 value scales (32-63 a copy)
          dma4(((lane & 16) ? P.v_scale : P.k_scale) + hb * bs + slot0 + (lane & 15), uniform(base + 32 * D));
        } else {
          // keys: LDS chunk p = 64 i + l is chunk (p % kCh) of slot r = p / kCh
          // and holds the row's chunk (p % kCh) ^ (r % kCh)
#pragma unroll
          for (int i = 0; i < D / 32; ++i) {
            const int pc = 64 * i + lane, r = pc / kCh, cc = (pc % kCh) ^ (r % kCh);
            dma16(kc8 + ((hb * bs + slot0 + r) * D + 8 * cc) * 2, uniform(base + 1024 * i));
          }
          // values: LDS chunk p = 64 i + l is half (p % 2) of dimension p / 2
#pragma unroll
          for (int i = 0; i < D / 32; ++i) {
            const int pc = 64 * i + lane;
            dma16(vc8 + ((hb * D + (pc >> 1)) * bs + slot0 + 8 * (pc & 1)) * 2, uniform(base + 32 * D + 1024 * i));
          }
        }
      };
      auto compute_tile = [&](int ti) {
        const uint8_t* sb = ring + (ti & (kRingStages - 1)) * kStageB;
        KT kr[NS];
        VTy vr[NJ];
        float4 ks = make_float4(1.f, 1.f, 1.f, 1.f), vs = ks;
        if constexpr (F8) {
#pragma unroll
          for (int k = 0; k < NS; ++k) kr[k] = *reinterpret_cast<const uint2*>(sb + (4 * k + lg) * 128 + 8 * l16);
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            vr[j] = *reinterpret_cast<const uint32_t*>(sb + 16 * D + 16 * (16 * j + l16) + 4 * lg);
          ks = *reinterpret_cast<const float4*>(sb + 32 * D + 16 * lg);
          vs = *reinterpret_cast<const float4*>(sb + 32 * D + 64 + 16 * lg);
        } else {
          // lane (slot l%16, dims 32 k + 8 (l/16) ..): chunk 4 k + l/16 of its slot
#pragma unroll
          for (int k = 0; k < NS; ++k)
            kr[k] = *reinterpret_cast<const KT*>(sb + 2 * D * l16 + 16 * ((4 * k + lg) ^ (l16 % kCh)));
          // lane (dimension 16 j + l%16, slots 4 (l/16) ..): 8 bytes
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            vr[j] = *reinterpret_cast<const VTy*>(sb + 32 * D + 32 * (16 * j + l16) + 8 * lg);
        }
        compute(t0 + (ti << 4), kr, vr, ks, vs);
      };
      // the previous item's trailing tiles (past its end, L2 hits) and the
      // next item's block ids and query land before this item's tiles, so
      // the waits below count this item's DMA exactly
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      if (next_item < total_items) fetch(next_item, nblk, nq);
#pragma unroll
      for (int c = 0; c < kRingStages - 1; ++c) dma_tile(c);
      for (int ti = 0; ti < n_tiles; ++ti) {
        dma_tile(ti + kRingStages - 1);            // into the stage of tile ti-1
        wait_vmcnt<(kRingStages - 1) * kOps>();    // tile ti has landed
        compute_tile(ti);
      }
    } else {
      // TPS tiles per pipeline stage: an FP8 tile is half the bytes of a bf16
      // one, so two are staged together to keep as many bytes in flight
      constexpr int TPS = F8 ? 2 : 1;
      KT ka[TPS][NS], kb[TPS][NS];
      VTy va[TPS][NJ], vb[TPS][NJ];
      float4 ksa[TPS], vsa[TPS], ksb[TPS], vsb[TPS];
      const int last = n_tiles - 1;
      auto issue_s = [&](int ti0, KT (&kr)[TPS][NS], VTy (&vr)[TPS][NJ], float4 (&ks)[TPS], float4 (&vs)[TPS]) {
  #pragma unroll
        for (int u = 0; u < TPS; ++u) issue(ti0 + u, kr[u], vr[u], ks[u], vs[u]);
      };
      auto compute_s = [&](int ti0, const KT (&kr)[TPS][NS], const VTy (&vr)[TPS][NJ], const float4 (&ks)[TPS],
                           const float4 (&vs)[TPS]) {
  #pragma unroll
        for (int u = 0; u < TPS; ++u) compute(t0 + ((ti0 + u) << 4), kr[u], vr[u], ks[u], vs[u]);
      };
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): see attn_split_kernel
      issue_s(0, ka, va, ksa, vsa);
      if (next_item < total_items) fetch(next_item, nblk, nq);
      for (int ti = 0; ti <= last; ti += 2 * TPS) {
        issue_s(ti + TPS, kb, vb, ksb, vsb);
        compute_s(ti, ka, va, ksa, vsa);
        issue_s(ti + 2 * TPS, ka, va, ksa, vsa);
        compute_s(ti + TPS, kb, vb, ksb, vsb);
      }
    }

    // row sums: add the four lanes of each row
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    // lane l holds O^T[16 j + 4 (l/16) + i][row l%16]
    if (l16 < nrow) {
      const size_t bh = (size_t)b * P.H_kv + h;
      if (ns == 1) {
        const int j = l16 / P.G, gi = l16 - (l16 / P.G) * P.G;
        uint16_t* orow = op + ((size_t)(b * P.Kq + j) * P.H_q + h * P.G + gi) * D + 4 * lg;
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
          const f32x4_t a = acc[jj] * inv;
          *reinterpret_cast<uint2*>(orow + 16 * jj) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
        }
      } else {
        const size_t pr = (bh * P.max_splits + s) * NR + l16;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
          *reinterpret_cast<f32x4_t*>(P.part_acc + pr * D + 16 * jj + 4 * lg) = acc[jj];
        if (lg == 0) { P.part_ml[2 * pr] = m; P.part_ml[2 * pr + 1] = lsum; }
      }
    }
    item = next_item;
    my_blk = nblk;
#pragma unroll
    for (int k = 0; k < NS; ++k) qf[k] = nq[k];
  }
}

// Merge the splits of each (stream, KV head, query row) that has more than
// one: o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, in split order.
// One wave per row: lane i holds split i's (m, l); each lane accumulates
// D/64 head dimensions.
template <typename T, int D, int NR>
__global__ __launch_bounds__(kThreads) void attn_combine_kernel(KParams P) {
  constexpr int DL = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= P.B * P.H_kv * P.nr) return;
  const int r = row % P.nr;
  const int bh = row / P.nr;
  const int b = bh / P.H_kv;
  const int h = bh - b * P.H_kv;
  const int ns = uniform(split_count(stream_len(P.kv_len[b], P), P));
  if (ns <= 1) return;
  const size_t base = (size_t)bh * P.max_splits * NR + r;

  const int j = r / P.G, gi = r - (r / P.G) * P.G;
  T* orow = static_cast<T*>(P.o) + ((size_t)(b * P.Kq + j) * P.H_q + h * P.G + gi) * D;
  if (ns <= 16) {
    // every split's (m, l) and accumulator loads issued together: one round
    // trip; the same arithmetic, in the same order, as the general form below
    const float mi = lane < ns ? P.part_ml[2 * (base + (size_t)lane * NR)] : kNegBig;
    const float li = lane < ns ? P.part_ml[2 * (base + (size_t)lane * NR) + 1] : 0.f;
    float v[16][DL];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float* a = P.part_acc + (base + (size_t)min(k, ns - 1) * NR) * D + lane;
#pragma unroll
      for (int e = 0; e < DL; ++e) v[k][e] = a[64 * e];
    }
    const float M = fmaxf(kNegBig, wave_max(mi));
    const float f = lane < ns ? __builtin_amdgcn_exp2f(mi - M) : 0.f;
    const float L = 0.f + wave_sum(f * li);
    float A[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) A[e] = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float fk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), k));
      if (k < ns) {
#pragma unroll
        for (int e = 0; e < DL; ++e) A[e] = fmaf(fk, v[k][e], A[e]);
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) store_out(orow + lane + 64 * e, A[e] * inv);
    return;
  }

  // (m, l) of up to 64 splits per lane-parallel pass; accumulators in
  // batches of 16 splits whose loads are all issued before any is used
  float M = kNegBig;
  for (int i0 = 0; i0 < ns; i0 += 64) {
    const int i = i0 + lane;
    const float mi = i < ns ? P.part_ml[2 * (base + (size_t)i * NR)] : kNegBig;
    M = fmaxf(M, wave_max(mi));
  }
  float L = 0.f, A[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) A[e] = 0.f;
  for (int i0 = 0; i0 < ns; i0 += 64) {
    const int i = i0 + lane;
    float f = 0.f, li = 0.f;
    if (i < ns) {
      f = __builtin_amdgcn_exp2f(P.part_ml[2 * (base + (size_t)i * NR)] - M);
      li = P.part_ml[2 * (base + (size_t)i * NR) + 1];
    }
    L += wave_sum(f * li);
    const int cnt = min(64, ns - i0);
    for (int k0 = 0; k0 < cnt; k0 += 16) {
      float v[16][DL];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int kk = min(k0 + k, cnt - 1);
        const float* a = P.part_acc + (base + (size_t)(i0 + kk) * NR) * D + lane;
#pragma unroll
        for (int e = 0; e < DL; ++e) v[k][e] = a[64 * e];
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float fk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), min(k0 + k, 63)));
        if (k0 + k < cnt) {
#pragma unroll
          for (int e = 0; e < DL; ++e) A[e] = fmaf(fk, v[k][e], A[e]);
        }
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int e = 0; e < DL; ++e) store_out(orow + lane + 64 * e, A[e] * inv);
}

int device_cus() {
  static std::atomic<int> cus[64];   // 0 until queried; calls may come from any host thread
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (!n) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename T, int D, int NR>
hipError_t launch_t(const KParams& P, int grid, hipStream_t s) {
  const bool exact = P.nr == NR;
  if (P.k_scale) {                       // FP8 cache: matrix-core kernel at every row count
    if constexpr (std::is_same<T, uint16_t>::value) {
      // up to kRingMaxB streams: tiles staged through an LDS ring
      if (P.B <= kRingMaxB && P.bs == 16)
        hipLaunchKernelGGL((attn_mfma_kernel<D, NR, 16, true, true>), dim3(grid), dim3(kThreads), 0, s, P);
      else if (P.B <= kRingMaxB)
        hipLaunchKernelGGL((attn_mfma_kernel<D, NR, 0, true, true>), dim3(grid), dim3(kThreads), 0, s, P);
      else if (P.bs == 16)
        hipLaunchKernelGGL((attn_mfma_kernel<D, NR, 16, true>), dim3(grid), dim3(kThreads), 0, s, P);
      else
        hipLaunchKernelGGL((attn_mfma_kernel<D, NR, 0, true>), dim3(grid), dim3(kThreads), 0, s, P);
    } else {
      return hipErrorInvalidValue;
    }
  } else if constexpr (std::is_same<T, uint16_t>::value && NR > 2) {
    if (P.B <= kRingMaxB && P.bs == 16)
      hipLaunchKernelGGL((attn_mfma_kernel<D, NR, 16, false, true>), dim3(grid), dim3(kThreads), 0, s, P);
    else if (P.B <= kRingMaxB)
      hipLaunchKernelGGL((attn_mfma_kernel<D, NR, 0, false, true>), dim3(grid), dim3(kThreads), 0, s, P);
    else if (P.bs == 16)
      hipLaunchKernelGGL((attn_mfma_kernel<D, NR, 16, false>), dim3(grid), dim3(kThreads), 0, s, P);
    else
      hipLaunchKernelGGL((attn_mfma_kernel<D, NR, 0, false>), dim3(grid), dim3(kThreads), 0, s, P);
  } else if (P.bs == 16 && exact)
    hipLaunchKernelGGL((attn_split_kernel<T, D, NR, 16, true>), dim3(grid), dim3(kThreads), 0, s, P);
  else if (P.bs == 16)
    hipLaunchKernelGGL((attn_split_kernel<T, D, NR, 16, false>), dim3(grid), dim3(kThreads), 0, s, P);
  else
    hipLaunchKernelGGL((attn_split_kernel<T, D, NR, 0, false>), dim3(grid), dim3(kThreads), 0, s, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P.max_splits <= 1) return e;
  const long rows = (long)P.B * P.H_kv * P.nr;
  hipLaunchKernelGGL((attn_combine_kernel<T, D, NR>), dim3((rows + kWaves - 1) / kWaves), dim3(kThreads), 0, s, P);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_nr(const KParams& P, int nr_tmpl, int grid, hipStream_t s) {
  switch (nr_tmpl) {
    case 1: return launch_t<T, D, 1>(P, grid, s);
    case 2: return launch_t<T, D, 2>(P, grid, s);
    case 4: return launch_t<T, D, 4>(P, grid, s);
    case 8: return launch_t<T, D, 8>(P, grid, s);
    case 12: return launch_t<T, D, 12>(P, grid, s);
    case 16: return launch_t<T, D, 16>(P, grid, s);
  }
  return hipErrorInvalidValue;
}


}  // namespace


hipError_t attention_scratch(void** ptr) {
  constexpr int kMaxDev = 64;
  static void* addr[kMaxDev] = {nullptr};
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  KParams P;
  P.q = a.q; P.kc = a.k_cache; P.vc = a.v_cache;
  P.k_scale = a.k_scale; P.v_scale = a.v_scale;
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
  // Three workgroups per CU are resident for the vector and bf16 kernels.  The
  // FP8 LDS-ring kernel fits two per CU; its grid is 6x the CUs, so that the
  // hardware hands later workgroups (the shorter items) to CUs as they free
  // up (256 streams: 177 against 180 us at 3x).
  const bool f8_ring = a.k_scale != nullptr && a.B <= kRingMaxB;
  const long cap_wg = (f8_ring ? 6L : 3L) * device_cus();
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
