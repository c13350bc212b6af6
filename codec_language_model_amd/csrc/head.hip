// Codebook logit projection: logits[r, v] = sum_k h[r, k] * W_{g(r)}[v, k]
// (TontaubeV1, audio head paragraph: a per-stage head onto that stage's
// codebook; codec paragraph for the 16,384 / 4,096 entry codebooks).
//
// bf16: matrix-core kernel.  A workgroup owns VT*16 codebook entries of one
// stage's W and up to 64 rows of that stage (rows are gathered by head id, in
// batch order), so each W byte is streamed from HBM once per 64 rows.  The
// products use v_mfma_f32_16x16x32_bf16 with W as the A operand (16 codebook
// entries x 32 k) and h as B (32 k x 16 rows): the accumulator lane l holds
// logits for row l%16 and 4 consecutive entries, which become one 16-byte
// store.  The four waves split the reduction (k) dimension; their partial
// tiles are summed in LDS in wave order, so the result is deterministic.
// Operands come straight from global memory with the next k-step's loads in
// flight; h (<= 64 rows) stays resident in L2 while W streams past it.
//
// fp32: a plain wave-per-row GEMV (used by the small fp32 workload).
#include "clm_device.h"
#include "clm_launch.h"

namespace clm {
namespace {

constexpr int kRowsPerWG = 64;

struct HeadP {
  const uint16_t* h;
  const uint16_t* W[8];
  const int32_t* head_id;
  float* logits;
  int G, M, d, V, row_chunks;
};

template <int VT>
__global__ __launch_bounds__(256) void head_mfma_kernel(HeadP P) {
  constexpr int NV = VT * 16;        // codebook entries per workgroup
  constexpr int LDW = NV + 4;        // padded LDS row (floats)
  __shared__ int s_rows[kRowsPerWG];
  __shared__ int s_cnt[4];
  __shared__ float s_red[4][kRowsPerWG][LDW];

  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int grp = blockIdx.y / P.row_chunks;
  const int rc = blockIdx.y - grp * P.row_chunks;
  const int v0 = blockIdx.x * NV;

  // ---- rows of this stage, chunk rc (batch order) ---------------------------
  int n_rows;
  if (P.G == 1) {
    n_rows = min(kRowsPerWG, P.M - rc * kRowsPerWG);
    if (tid < kRowsPerWG) s_rows[tid] = min(rc * kRowsPerWG + tid, P.M - 1);
    __syncthreads();
  } else {
    const int per = (P.M + 255) / 256;
    const int r0 = tid * per;
    int cnt = 0;
    for (int k = 0; k < per; ++k) {
      int r = r0 + k;
      if (r < P.M && clampi(P.head_id[r], 0, P.G - 1) == grp) ++cnt;
    }
    int incl = wave_incl_scan_i(cnt, lane);
    if (lane == 63) s_cnt[w] = incl;
    __syncthreads();
    int rank = incl - cnt;
    for (int i = 0; i < w; ++i) rank += s_cnt[i];
    const int total = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
    for (int k = 0; k < per; ++k) {
      int r = r0 + k;
      if (r < P.M && clampi(P.head_id[r], 0, P.G - 1) == grp) {
        const int slot = rank - rc * kRowsPerWG;
        if (slot >= 0 && slot < kRowsPerWG) s_rows[slot] = r;
        ++rank;
      }
    }
    n_rows = min(kRowsPerWG, total - rc * kRowsPerWG);
    __syncthreads();
    if (n_rows > 0 && tid >= n_rows && tid < kRowsPerWG) s_rows[tid] = s_rows[0];
    __syncthreads();
  }
  n_rows = uniform(n_rows);
  if (n_rows <= 0) return;
  const int n_rt = (n_rows + 15) >> 4;

  const uint16_t* __restrict__ Wg = P.W[grp];
  const int kq = P.d >> 2;              // k range per wave
  const int kb = w * kq;
  const int l16 = lane & 15, lg = lane >> 4;

  const uint16_t* aptr[VT];
#pragma unroll
  for (int vt = 0; vt < VT; ++vt) {
    const int v = min(v0 + vt * 16 + l16, P.V - 1);
    aptr[vt] = Wg + (size_t)v * P.d + kb + lg * 8;
  }
  const uint16_t* bptr[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) bptr[rt] = P.h + (size_t)s_rows[rt * 16 + l16] * P.d + kb + lg * 8;

  f32x4_t acc[VT][4];
#pragma unroll
  for (int vt = 0; vt < VT; ++vt)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) acc[vt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  bf16x8_t a[VT], bb[4];
#pragma unroll
  for (int vt = 0; vt < VT; ++vt) a[vt] = *reinterpret_cast<const bf16x8_t*>(aptr[vt]);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
    if (rt < n_rt) bb[rt] = *reinterpret_cast<const bf16x8_t*>(bptr[rt]);

  for (int k = 0; k < kq; k += 32) {
    bf16x8_t na[VT], nb[4];
    if (k + 32 < kq) {
#pragma unroll
      for (int vt = 0; vt < VT; ++vt) na[vt] = *reinterpret_cast<const bf16x8_t*>(aptr[vt] + k + 32);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        if (rt < n_rt) nb[rt] = *reinterpret_cast<const bf16x8_t*>(bptr[rt] + k + 32);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (rt < n_rt) {
#pragma unroll
        for (int vt = 0; vt < VT; ++vt)
          acc[vt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[vt], bb[rt], acc[vt][rt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) a[vt] = na[vt];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) bb[rt] = nb[rt];
  }

  // ---- sum the four k-slices in wave order and store ------------------------
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    if (rt < n_rt) {
#pragma unroll
      for (int vt = 0; vt < VT; ++vt)
        *reinterpret_cast<f32x4_t*>(&s_red[w][rt * 16 + l16][vt * 16 + lg * 4]) = acc[vt][rt];
    }
  }
  __syncthreads();
  for (int e = tid; e < n_rows * NV; e += 256) {
    const int rl = e / NV, vl = e - (e / NV) * NV;
    const int v = v0 + vl;
    if (v < P.V) {
      const float s = ((s_red[0][rl][vl] + s_red[1][rl][vl]) + s_red[2][rl][vl]) + s_red[3][rl][vl];
      P.logits[(size_t)s_rows[rl] * P.V + v] = s;
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
    P.G = a.G; P.M = a.M; P.d = a.d; P.V = a.V;
    P.row_chunks = (a.M + kRowsPerWG - 1) / kRowsPerWG;
    // Enough workgroups to cover the chip: 64-entry tiles when that already
    // gives >= 512 workgroups, else 32-entry tiles.
    const long wg64 = (long)((a.V + 63) / 64) * a.G * P.row_chunks;
    if (wg64 >= 512) {
      dim3 grid((a.V + 63) / 64, a.G * P.row_chunks);
      hipLaunchKernelGGL(head_mfma_kernel<4>, grid, dim3(256), 0, s, P);
    } else {
      dim3 grid((a.V + 31) / 32, a.G * P.row_chunks);
      hipLaunchKernelGGL(head_mfma_kernel<2>, grid, dim3(256), 0, s, P);
    }
    return hipGetLastError();
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
