// Codebook logit projection: logits[r, v] = sum_k h[r, k] * W_{g(r)}[v, k]
// (TontaubeV1, audio head paragraph: a per-stage head onto that stage's
// codebook; codec paragraph for the 16,384 / 4,096 entry codebooks).
//
// bf16: matrix-core kernel with v_mfma_f32_16x16x32_bf16.  A workgroup owns
// a tile of NV codebook entries of one stage's W and MR rows of that stage
// (rows are gathered by head id, in batch order) and walks k in chunks of 64.
// Each chunk of both operands goes from global memory straight into LDS with
// the global-to-LDS DMA loads (every instruction moves 8 whole 128-byte row
// pieces; pieces are XOR-swizzled by row so the matrix cores' 16-byte operand
// reads are bank-conflict free), three chunks in flight while one is
// multiplied.  The four waves are laid out 2 (entries) x 2 (rows) and write
// their logits directly, 4 consecutive entries per lane.  MR in {32, 64, 128}
// pads the fewest rows; NV in {128, 64, 32} is the widest that still gives
// 256 workgroups.  When a stage has several row chunks they read the same W
// tile: the 1-D grid is laid out so those workgroups sit on one XCD (the
// hardware deals workgroup i to XCD i % 8) and run together, so W comes from
// HBM once and from that XCD's L2 after.  W is read once per call for up to
// 128 rows.
//
// Two-layer head (TontaubeV1, audio head paragraph: widen to 4,096, Mish,
// project): the same kernel with a Mish epilogue that stores the bf16
// activation, then the plain kernel on that activation.
//
// fp32: a plain wave-per-row GEMV (used by the small fp32 workload).
#include "clm_device.h"
#include "clm_launch.h"

namespace clm {
namespace {

constexpr int kXcds = 8;

struct HeadP {
  const uint16_t* h;
  const uint16_t* W[8];
  const int32_t* head_id;
  float* logits;
  uint16_t* act;    // MISH epilogue: bf16 activations [M, V]
  int G, M, d, V, row_chunks, nvt, nvt_pad;
};

// Rows of stage grp that fall in row chunk rc (MR rows each, batch order) into
// s_rows; slots past the last row repeat a valid row so loads stay in bounds.
// Returns the chunk's row count (<= 0: nothing to do), the same in all lanes.
template <int MR, int NT>
__device__ __forceinline__ int gather_rows(const HeadP& P, int grp, int rc, int* s_rows, int* s_cnt,
                                           int tid, int lane, int w) {
  constexpr int NW = NT / 64;
  int n_rows;
  if (P.G == 1) {
    n_rows = min(MR, P.M - rc * MR);
    for (int i = tid; i < MR; i += NT) s_rows[i] = min(rc * MR + i, P.M - 1);
    __syncthreads();
  } else {
    const int per = (P.M + NT - 1) / NT;
    const int r0 = tid * per;
    int cnt = 0;
    for (int k = 0; k < per; ++k) {
      const int r = r0 + k;
      if (r < P.M && clampi(P.head_id[r], 0, P.G - 1) == grp) ++cnt;
    }
    const int incl = wave_incl_scan_i(cnt);
    if (lane == 63) s_cnt[w] = incl;
    __syncthreads();
    int rank = incl - cnt;
    int total = 0;
    for (int i = 0; i < NW; ++i) {
      if (i < w) rank += s_cnt[i];
      total += s_cnt[i];
    }
    for (int k = 0; k < per; ++k) {
      const int r = r0 + k;
      if (r < P.M && clampi(P.head_id[r], 0, P.G - 1) == grp) {
        const int slot = rank - rc * MR;
        if (slot >= 0 && slot < MR) s_rows[slot] = r;
        ++rank;
      }
    }
    n_rows = min(MR, total - rc * MR);
    __syncthreads();
    for (int i = tid; i < MR; i += NT)
      if (n_rows > 0 && i >= n_rows) s_rows[i] = s_rows[0];
    __syncthreads();
  }
  return uniform(n_rows);
}

// Mish(x) = x * tanh(softplus(x)), written with y = 1 + e^x as
// x * (y^2 - 1) / (y^2 + 1) = x * n (n + 2) / (n (n + 2) + 2), n = e^x; for
// x > 20 the ratio is 1 in fp32 (and n^2 would overflow past x = 44).
__device__ __forceinline__ float mish_f(float x) {
  if (x > 20.f) return x;
  const float n = expf(x);
  const float t = n * (n + 2.f);
  return x * t / (t + 2.f);
}

// LDS fed by DMA: S stages of one 64-k chunk each, holding NV codebook rows
// then MR h rows (128 bytes per row, the 16-byte pieces XOR-swizzled by row
// so the operand reads are bank-conflict free).  Each DMA instruction fills
// 8 whole rows (1 KiB), lane l taking the piece that belongs in slot l % 8;
// S - 1 chunks are in flight while one is multiplied, one barrier per chunk.
//
// The products are always accumulated as two chains: the even 32-k substeps
// of the chunks (k = 64c .. 64c+31) in one set of accumulators and the odd
// ones (k = 64c+32 .. 64c+63) in another, and the two are added once at the
// end.  With NW = 8 waves the two chains belong to two groups of 4 waves,
// which gives each SIMD two waves to overlap operand reads, DMA and matrix
// products (the second group's sums reach the first through LDS); with
// NW = 4 each wave keeps both chains.  Every tile shape and wave count thus
// produces the same bits for a given row, whatever else is in the batch.
// Within a group the 4 waves are laid out 2 (entries) x 2 (rows), each
// owning NV/2 entries x MR/2 rows.
template <int NV, int MR, int S, int NW, bool MISH>
__global__ __launch_bounds__(NW * 64) void head_dma_kernel(HeadP P) {
  constexpr int KC = 64;                      // k per chunk
  constexpr int ROWS = NV + MR;               // LDS rows per stage
  constexpr int STAGE = ROWS * KC;            // bf16 elements per stage
  constexpr int NT = NW * 64;
  constexpr int NI = ROWS / (8 * NW);         // DMA instructions per wave per chunk
  constexpr int VTW = NV / 32, RTW = MR / 32; // 16-wide tiles per wave
  constexpr int NCH = NW == 8 ? 1 : 2;        // chains (substeps) per wave
  static_assert(ROWS % (8 * NW) == 0, "rows per stage");
  static_assert(S >= 2 && (S - 2) * NI < 64, "pipeline depth");
  static_assert(NW == 4 || VTW * RTW * 4 * 64 * 16 <= S * STAGE * 2, "chain sums fit the ring");
  __shared__ int s_rows[MR];
  __shared__ int s_cnt[NW];
  __shared__ __attribute__((aligned(1024))) uint16_t s_buf[S * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int grp_w = NW == 8 ? (w >> 2) : 0, wq = w & 3;
  const int per_grp = P.nvt_pad * P.row_chunks;
  const int grp = blockIdx.x / per_grp;
  const int id = blockIdx.x - grp * per_grp;
  const int super = id / (kXcds * P.row_chunks);
  const int rem = id - super * kXcds * P.row_chunks;
  const int rc = rem / kXcds;
  const int vt = super * kXcds + (rem - rc * kXcds);
  if (vt >= P.nvt) return;
  const int v0 = vt * NV;
  const int n_rows = gather_rows<MR, NT>(P, grp, rc, s_rows, s_cnt, tid, lane, w);
  if (n_rows <= 0) return;

  const uint16_t* __restrict__ Wg = P.W[grp];
  const int nch = P.d / KC;
  // DMA instruction j of wave w fills rows 8r..8r+7, r = NW j + w; lane l
  // reads row 8r + l/8, piece (l % 8) ^ (l / 8) (row & 7 == l / 8).
  const uint16_t* src[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int R = 8 * (NW * j + w) + (lane >> 3);
    const int piece = (lane & 7) ^ (lane >> 3);
    const uint16_t* row = R < NV ? Wg + (size_t)min(v0 + R, P.V - 1) * P.d
                                 : P.h + (size_t)s_rows[R - NV] * P.d;
    src[j] = row + piece * 8;
  }
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(s_buf);
  auto issue = [&](int chunk, int stage) __attribute__((always_inline)) {
    const uint32_t base = lds0 + (uint32_t)(stage * STAGE * 2);
#pragma unroll
    for (int j = 0; j < NI; ++j)
      dma16(src[j] + chunk * KC, uniform(base + (uint32_t)((NW * j + w) * 1024)));
  };

  const int wv = wq & 1, wr = wq >> 1;
  const int l16 = lane & 15, lg = lane >> 4;
  int aoff[NCH][VTW], boff[NCH][RTW];
#pragma unroll
  for (int s = 0; s < NCH; ++s) {
    const int c = 4 * (NW == 8 ? grp_w : s) + lg;
#pragma unroll
    for (int t = 0; t < VTW; ++t) {
      const int R = (NV / 2) * wv + 16 * t + l16;
      aoff[s][t] = R * KC + ((c ^ (R & 7)) << 3);
    }
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      const int R = NV + wr * (MR / 2) + 16 * t + l16;
      boff[s][t] = R * KC + ((c ^ (R & 7)) << 3);
    }
  }
  f32x4_t acc[NCH][VTW][RTW];
#pragma unroll
  for (int s = 0; s < NCH; ++s)
#pragma unroll
    for (int a = 0; a < VTW; ++a)
#pragma unroll
      for (int t = 0; t < RTW; ++t) acc[s][a][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int stage) __attribute__((always_inline)) {
    const uint16_t* sb = s_buf + stage * STAGE;
#pragma unroll
    for (int s = 0; s < NCH; ++s) {
      bf16x8_t A[VTW], Bm[RTW];
#pragma unroll
      for (int t = 0; t < VTW; ++t) A[t] = *reinterpret_cast<const bf16x8_t*>(sb + aoff[s][t]);
#pragma unroll
      for (int t = 0; t < RTW; ++t) Bm[t] = *reinterpret_cast<const bf16x8_t*>(sb + boff[s][t]);
#pragma unroll
      for (int t = 0; t < RTW; ++t)
#pragma unroll
        for (int a = 0; a < VTW; ++a)
          acc[s][a][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[a], Bm[t], acc[s][a][t], 0, 0, 0);
    }
  };

  // Chunk c lives in stage c % S.  At the top of iteration i, chunks
  // i+1 .. i+S-2 may still be in flight ((S-2)*NI loads of this wave); near
  // the end fewer were issued, so wait for all.  The barrier then also
  // retires every wave's reads of stage (i-1) % S, which is refilled next.
#pragma unroll
  for (int c = 0; c < S - 1; ++c)
    if (c < nch) issue(c, c);
  int stage = 0;
  for (int i = 0; i < nch; ++i) {
    if (i + S - 2 < nch) wait_vmcnt<(S - 2) * NI>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (i + S - 1 < nch) issue(i + S - 1, stage == 0 ? S - 1 : stage - 1);
    compute(stage);
    stage = stage == S - 1 ? 0 : stage + 1;
  }

  // even chain + odd chain
  f32x4_t tot[VTW][RTW];
  if constexpr (NW == 8) {
    __syncthreads();                          // every wave is done with the ring
    f32x4_t* red = reinterpret_cast<f32x4_t*>(s_buf);
    if (grp_w == 1) {
#pragma unroll
      for (int a = 0; a < VTW; ++a)
#pragma unroll
        for (int t = 0; t < RTW; ++t) red[((wq * VTW + a) * RTW + t) * 64 + lane] = acc[0][a][t];
    }
    __syncthreads();
    if (grp_w == 1) return;
#pragma unroll
    for (int a = 0; a < VTW; ++a)
#pragma unroll
      for (int t = 0; t < RTW; ++t) tot[a][t] = acc[0][a][t] + red[((wq * VTW + a) * RTW + t) * 64 + lane];
  } else {
#pragma unroll
    for (int a = 0; a < VTW; ++a)
#pragma unroll
      for (int t = 0; t < RTW; ++t) tot[a][t] = acc[0][a][t] + acc[NCH - 1][a][t];
  }

#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    const int R = wr * (MR / 2) + 16 * t + l16;
    if (R < n_rows) {
      if constexpr (MISH) {
        uint16_t* orow = P.act + (size_t)s_rows[R] * P.V;
#pragma unroll
        for (int a = 0; a < VTW; ++a) {
          const int v = v0 + (NV / 2) * wv + 16 * a + 4 * lg;
          const f32x4_t y = {mish_f(tot[a][t][0]), mish_f(tot[a][t][1]), mish_f(tot[a][t][2]),
                             mish_f(tot[a][t][3])};
          if (v + 3 < P.V) {
            *reinterpret_cast<uint2*>(orow + v) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (v + e < P.V) orow[v + e] = f32_to_bf16(y[e]);
          }
        }
      } else {
        float* orow = P.logits + (size_t)s_rows[R] * P.V;
#pragma unroll
        for (int a = 0; a < VTW; ++a) {
          const int v = v0 + (NV / 2) * wv + 16 * a + 4 * lg;
          if (v + 3 < P.V) {
            *reinterpret_cast<f32x4_t*>(orow + v) = tot[a][t];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (v + e < P.V) orow[v + e] = tot[a][t][e];
          }
        }
      }
    }
  }
}

struct GemvP {
  const float* h;
  const float* W[8];
  const int32_t* head_id;
  float* logits;
  int G, M, d, V;
};

// One wave per codebook entry, all rows; d % 4 == 0.
__global__ __launch_bounds__(256) void head_gemv_f32_kernel(GemvP P) {
  const int lane = threadIdx.x & 63;
  const int v = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (v >= P.V) return;
  for (int r = 0; r < P.M; ++r) {
    const int g = P.G == 1 ? 0 : clampi(P.head_id[r], 0, P.G - 1);
    const float* wrow = P.W[g] + (size_t)v * P.d;
    const float* hrow = P.h + (size_t)r * P.d;
    float acc = 0.f;
    for (int k = lane * 4; k < P.d; k += 256) {
      const float4 x = *reinterpret_cast<const float4*>(wrow + k);
      const float4 y = *reinterpret_cast<const float4*>(hrow + k);
      acc = fmaf(x.x, y.x, acc);
      acc = fmaf(x.y, y.y, acc);
      acc = fmaf(x.z, y.z, acc);
      acc = fmaf(x.w, y.w, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) P.logits[(size_t)r * P.V + v] = acc;
  }
}

}  // namespace


hipError_t launch_codebook_head(const HeadArgs& a, hipStream_t s) {
  if (a.bf16) {
    HeadP P;
    P.h = static_cast<const uint16_t*>(a.h);
    for (int g = 0; g < 8; ++g) P.W[g] = static_cast<const uint16_t*>(g < a.G ? a.W[g] : a.W[0]);
    P.head_id = a.head_id;
    P.logits = a.logits;
    P.act = a.act;
    P.G = a.G; P.M = a.M; P.d = a.d; P.V = a.V;
    const HeadPlan hp = plan_codebook_head(a.M, a.V, a.G);
    P.row_chunks = hp.row_chunks;
    P.nvt = hp.nvt;
    P.nvt_pad = hp.nvt_pad;
    const dim3 g((unsigned)((long)P.nvt_pad * P.row_chunks * a.G)), b(hp.nw * 64);
#define CLM_HEAD_DMA(NV_, MR_)                                                                         \
    if (hp.nv == NV_ && hp.mr == MR_) {                                                                \
      constexpr int NW_ = (MR_ >= 96 && (NV_ + MR_) % 64 == 0) ? 8 : 4;                                \
      if (a.act) hipLaunchKernelGGL((head_dma_kernel<NV_, MR_, 4, NW_, true>), g, b, 0, s, P);         \
      else hipLaunchKernelGGL((head_dma_kernel<NV_, MR_, 4, NW_, false>), g, b, 0, s, P);              \
      return hipGetLastError();                                                                        \
    }
    CLM_HEAD_DMA(128, 128) CLM_HEAD_DMA(128, 96) CLM_HEAD_DMA(128, 64) CLM_HEAD_DMA(128, 32)
    CLM_HEAD_DMA(64, 128) CLM_HEAD_DMA(64, 96) CLM_HEAD_DMA(64, 64) CLM_HEAD_DMA(64, 32)
    CLM_HEAD_DMA(32, 128) CLM_HEAD_DMA(32, 96) CLM_HEAD_DMA(32, 64) CLM_HEAD_DMA(32, 32)
#undef CLM_HEAD_DMA
    return hipErrorInvalidValue;
  }
  GemvP P;
  P.h = static_cast<const float*>(a.h);
  for (int g = 0; g < 8; ++g) P.W[g] = static_cast<const float*>(g < a.G ? a.W[g] : a.W[0]);
  P.head_id = a.head_id;
  P.logits = a.logits;
  P.G = a.G; P.M = a.M; P.d = a.d; P.V = a.V;
  hipLaunchKernelGGL(head_gemv_f32_kernel, dim3((a.V + 3) / 4), dim3(256), 0, s, P);
  return hipGetLastError();
}

}  // namespace clm
