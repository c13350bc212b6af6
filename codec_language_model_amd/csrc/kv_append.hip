// Paged KV append (Optimizing Streaming Text-to-Speech Models ..., "Dynamic
// Token-Level Batching": a static pool of fixed-size token blocks).
// One workgroup per (stream, KV head): key rows are copied as 16-byte chunks
// into their [bs, D] slot rows; value rows are scattered into the transposed
// [D, bs] block layout, one element per head dimension.
#include "clm_device.h"
#include "clm_launch.h"

namespace clm {
namespace {

struct AppendP {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* bt;
  const int32_t* len_before;
  int max_blocks, T_new, H_kv, bs, num_blocks;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendP P) {
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int CH = D / VE;
  const int b = blockIdx.x / P.H_kv;
  const int h = blockIdx.x - b * P.H_kv;
  const int lb = P.len_before[b];
  const int32_t* bt_row = P.bt + (size_t)b * P.max_blocks;
  const T* kn = static_cast<const T*>(P.k_new);
  const T* vn = static_cast<const T*>(P.v_new);
  T* kc = static_cast<T*>(P.k_cache);
  T* vc = static_cast<T*>(P.v_cache);

  // One pass over the key chunks (16 bytes) and then the value elements of
  // the new rows.  The source load does not depend on the destination, so
  // it is issued before the page lookup (len_before, then the block table).
  const int nk = P.T_new * CH;
  const int n_all = nk + P.T_new * D;
  for (int e = threadIdx.x; e < n_all; e += blockDim.x) {
    const bool is_k = e < nk;
    const int t = is_k ? e / CH : (e - nk) / D;
    const int part = is_k ? e - t * CH : (e - nk) - t * D;   // key chunk or value dimension
    const size_t row = ((size_t)(b * P.T_new + t) * P.H_kv + h) * D;
    uint4 k4 = make_uint4(0u, 0u, 0u, 0u);
    T v1 = T();
    if (is_k) k4 = *reinterpret_cast<const uint4*>(kn + row + part * VE);
    else v1 = vn[row + part];
    const int pos = lb + t;
    if (pos < 0) continue;
    const int page = pos / P.bs;
    if (page >= P.max_blocks) continue;
    const int blk = bt_row[page];
    if (blk < 0 || blk >= P.num_blocks) continue;
    const int slot = pos - page * P.bs;
    if (is_k)
      *reinterpret_cast<uint4*>(kc + (((size_t)blk * P.H_kv + h) * P.bs + slot) * D + part * VE) = k4;
    else
      vc[(((size_t)blk * P.H_kv + h) * D + part) * P.bs + slot] = v1;
  }
}

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ void from_f(float x, float* p) { *p = x; }
__device__ __forceinline__ void from_f(float x, uint16_t* p) { *p = f32_to_bf16(x); }

// Rotary embedding at logical positions fused with the append (TontaubeV1:
// positions are logical coordinates and only their differences matter; the
// speculative-decoding blog's engine fuses the rotary embedding with the KV
// cache write).  Per (stream, KV head) and new token t at logical position
// p = positions[b, t]: angles a_i = p * base^(-2i/D) in fp64 (p * theta in
// fp32 would be off by ~1e-3 rad at positions of 10^4), then pairs (i, i+D/2)
// of the key row are rotated on their way into the cache, the value row is
// copied as in the plain append, and the G query heads of this KV head are
// rotated in place.
struct RopeP {
  AppendP a;
  void* q;
  const int32_t* positions;
  int H_q, G;
  double log_base;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_append_kernel(RopeP R) {
  constexpr int HALF = D / 2;
  const AppendP& P = R.a;
  __shared__ float s_cos[HALF], s_sin[HALF];
  const int b = blockIdx.x / P.H_kv;
  const int h = blockIdx.x - b * P.H_kv;
  const int lb = P.len_before[b];
  const int32_t* bt_row = P.bt + (size_t)b * P.max_blocks;
  const T* kn = static_cast<const T*>(P.k_new);
  const T* vn = static_cast<const T*>(P.v_new);
  T* kc = static_cast<T*>(P.k_cache);
  T* vc = static_cast<T*>(P.v_cache);
  T* qp = static_cast<T*>(R.q);

  for (int t = 0; t < P.T_new; ++t) {
    const int p = R.positions[b * P.T_new + t];
    __syncthreads();                       // previous token's readers are done
    if (threadIdx.x < HALF) {
      const double th = exp(-2.0 * (double)threadIdx.x / (double)D * R.log_base);
      const double ang = (double)p * th;
      s_cos[threadIdx.x] = (float)cos(ang);
      s_sin[threadIdx.x] = (float)sin(ang);
    }
    __syncthreads();
    // the G query heads of this KV head, rotated in place
    for (int e = threadIdx.x; e < R.G * HALF; e += blockDim.x) {
      const int gi = e / HALF, i = e - (e / HALF) * HALF;
      T* qrow = qp + ((size_t)(b * P.T_new + t) * R.H_q + h * R.G + gi) * D;
      const float x0 = to_f(qrow[i]), x1 = to_f(qrow[i + HALF]);
      from_f(x0 * s_cos[i] - x1 * s_sin[i], qrow + i);
      from_f(x0 * s_sin[i] + x1 * s_cos[i], qrow + i + HALF);
    }
    const int pos = lb + t;
    if (pos < 0) continue;
    const int page = pos / P.bs;
    if (page >= P.max_blocks) continue;
    const int blk = bt_row[page];
    if (blk < 0 || blk >= P.num_blocks) continue;
    const int slot = pos - page * P.bs;
    const T* krow = kn + ((size_t)(b * P.T_new + t) * P.H_kv + h) * D;
    T* kdst = kc + (((size_t)blk * P.H_kv + h) * P.bs + slot) * D;
    for (int i = threadIdx.x; i < HALF; i += blockDim.x) {
      const float x0 = to_f(krow[i]), x1 = to_f(krow[i + HALF]);
      from_f(x0 * s_cos[i] - x1 * s_sin[i], kdst + i);
      from_f(x0 * s_sin[i] + x1 * s_cos[i], kdst + i + HALF);
    }
    for (int d = threadIdx.x; d < D; d += blockDim.x)
      vc[(((size_t)blk * P.H_kv + h) * D + d) * P.bs + slot] = vn[((size_t)(b * P.T_new + t) * P.H_kv + h) * D + d];
  }
}

template <typename T, int D>
hipError_t go_rope(const RopeP& R, int grid, hipStream_t s) {
  hipLaunchKernelGGL((rope_append_kernel<T, D>), dim3(grid), dim3(256), 0, s, R);
  return hipGetLastError();
}

// ---- FP8 (E4M3) cache: one scale per (token, KV head) row --------------------
// E4M3: 4 exponent bits (bias 7), 3 mantissa bits, largest 448, subnormals
// m * 2^-9.  Encoding of |x| <= 448, round to nearest, ties to the even code;
// the sign bit is x's (so -0 gives 0x80).
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a < 0.015625f) {                            // below 2^-6: subnormal step 2^-9
    const int m = (int)rintf(a * 512.0f);         // exact scaling; rint is round-half-even
    return sign | (uint32_t)m;                    // m == 8 is 2^-6, code 0x08
  }
  uint32_t u = __float_as_uint(a);
  u += 0x7FFFFu + ((u >> 20) & 1u);               // round the fp32 mantissa at bit 20, ties to even
  const int e = (int)(u >> 23) - 127 + 7;         // 1 .. 15
  return sign | ((uint32_t)e << 3) | ((u >> 20) & 7u);
}

// One wave quantizes one D-wide row held as D/64 values per lane: scale =
// max|x| / 448 (1 for an all-zero row), codes of x / scale clamped to +-448.
template <int D>
__device__ __forceinline__ float quantize_row(const float (&x)[D / 64], uint32_t (&code)[D / 64]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = wave_max(amax);
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) code[i] = e4m3_rne(fminf(fmaxf(x[i] / scale, -448.0f), 448.0f));
  return scale;
}

struct Fp8AppendP {
  AppendP a;
  float* k_scale;     // [num_blocks, H_kv, bs]
  float* v_scale;
  uint16_t* q;        // ROPE: [B, T_new, H_q, D] bf16, rotated in place
  const int32_t* positions;
  int H_q, G;
  double log_base;
};

// cos and sin of pair i's angle at logical position p, with the very
// expressions of rope_append_kernel (fp64, then fp32).
template <int D>
__device__ __forceinline__ void rope_cs(int p, int i, double log_base, float& c, float& s) {
  const double th = exp(-2.0 * (double)i / (double)D * log_base);
  const double ang = (double)p * th;
  c = (float)cos(ang);
  s = (float)sin(ang);
}

// The pair partner of the value this lane holds in slot k: lane l holds
// dimensions l + 64k, so at D = 128 the pair (i, i + 64) sits in one lane and
// at D = 64 the pair (i, i + 32) sits in lanes i and i + 32.
template <int D>
__device__ __forceinline__ void rope_row(float (&x)[D / 64], int lane, float c, float s) {
  if constexpr (D == 128) {
    const float x0 = x[0], x1 = x[1];
    x[0] = x0 * c - x1 * s;
    x[1] = x0 * s + x1 * c;
  } else {
    const float other = __shfl_xor(x[0], 32, 64);
    x[0] = lane < 32 ? x[0] * c - other * s : other * s + x[0] * c;
  }
}

// One workgroup of 2 waves per (stream, KV head): wave 0 quantizes and writes
// the key row of each new token, wave 1 the value row (transposed block).
// ROPE: wave 0 rotates the key row (fp32, from its bf16 values) before
// quantizing it, and wave 1 rotates the G query rows of this KV head in
// place after writing the value row.
template <int D, bool ROPE>
__global__ __launch_bounds__(128) void fp8_append_kernel(Fp8AppendP F) {
  const AppendP& P = F.a;
  const int b = blockIdx.x / P.H_kv;
  const int h = blockIdx.x - b * P.H_kv;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lb = P.len_before[b];
  const int32_t* bt_row = P.bt + (size_t)b * P.max_blocks;
  const uint16_t* src = static_cast<const uint16_t*>(w == 0 ? P.k_new : P.v_new);
  uint8_t* kc = static_cast<uint8_t*>(P.k_cache);
  uint8_t* vc = static_cast<uint8_t*>(P.v_cache);
  for (int t = 0; t < P.T_new; ++t) {
    // the row and its quantization do not depend on where it goes: load and
    // encode it while len_before and then the block table are looked up
    const uint16_t* row = src + ((size_t)(b * P.T_new + t) * P.H_kv + h) * D;
    float x[D / 64];
    uint32_t code[D / 64];
#pragma unroll
    for (int i = 0; i < D / 64; ++i) x[i] = bf16_to_f32(row[lane + 64 * i]);
    float rc = 1.f, rs = 0.f;
    if constexpr (ROPE) {
      rope_cs<D>(F.positions[b * P.T_new + t], lane % (D / 2), F.log_base, rc, rs);
      if (w == 0) rope_row<D>(x, lane, rc, rs);
    }
    const float scale = quantize_row<D>(x, code);
    if constexpr (ROPE) {
      if (w == 1) {
        // the G query heads of this KV head, in place (rope_append_kernel's arithmetic)
        for (int gi = 0; gi < F.G; ++gi) {
          uint16_t* qrow = F.q + ((size_t)(b * P.T_new + t) * F.H_q + h * F.G + gi) * D;
          if (lane < D / 2) {
            const int i = lane;
            const float x0 = bf16_to_f32(qrow[i]), x1 = bf16_to_f32(qrow[i + D / 2]);
            qrow[i] = f32_to_bf16(x0 * rc - x1 * rs);
            qrow[i + D / 2] = f32_to_bf16(x0 * rs + x1 * rc);
          }
        }
      }
    }
    const int pos = lb + t;
    if (pos < 0) continue;
    const int page = pos / P.bs;
    if (page >= P.max_blocks) continue;
    const int blk = bt_row[page];
    if (blk < 0 || blk >= P.num_blocks) continue;
    const int slot = pos - page * P.bs;
    const size_t hb = (size_t)blk * P.H_kv + h;
    if (w == 0) {
      // keys in 8-dimension groups: [block][head][d / 8][slot][d % 8]
#pragma unroll
      for (int i = 0; i < D / 64; ++i) {
        const int d = lane + 64 * i;
        kc[((hb * (D / 8) + (d >> 3)) * P.bs + slot) * 8 + (d & 7)] = (uint8_t)code[i];
      }
      if (lane == 0) F.k_scale[hb * P.bs + slot] = scale;
    } else {
#pragma unroll
      for (int i = 0; i < D / 64; ++i) vc[(hb * D + lane + 64 * i) * P.bs + slot] = (uint8_t)code[i];
      if (lane == 0) F.v_scale[hb * P.bs + slot] = scale;
    }
  }
}

template <typename T, int D>
hipError_t go(const AppendP& P, int grid, hipStream_t s) {
  hipLaunchKernelGGL((kv_append_kernel<T, D>), dim3(grid), dim3(256), 0, s, P);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s) {
  AppendP P{a.k_new, a.v_new, a.k_cache, a.v_cache, a.block_table, a.len_before,
            a.max_blocks, a.T_new, a.H_kv, a.block_size, a.num_blocks};
  const int grid = a.B * a.H_kv;
  if (a.bf16) {
    if (a.D == 128) return go<uint16_t, 128>(P, grid, s);
    if (a.D == 64) return go<uint16_t, 64>(P, grid, s);
  } else {
    if (a.D == 128) return go<float, 128>(P, grid, s);
    if (a.D == 64) return go<float, 64>(P, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace clm

namespace clm {

hipError_t launch_rope_kv_append(const RopeAppendArgs& a, hipStream_t s) {
  RopeP R;
  R.a = AppendP{a.k_new, a.v_new, a.k_cache, a.v_cache, a.block_table, a.len_before,
                a.max_blocks, a.T_new, a.H_kv, a.block_size, a.num_blocks};
  R.q = a.q;
  R.positions = a.positions;
  R.H_q = a.H_q;
  R.G = a.H_q / a.H_kv;
  R.log_base = log((double)a.rope_base);
  const int grid = a.B * a.H_kv;
  if (a.bf16) {
    if (a.D == 128) return go_rope<uint16_t, 128>(R, grid, s);
    if (a.D == 64) return go_rope<uint16_t, 64>(R, grid, s);
  } else {
    if (a.D == 128) return go_rope<float, 128>(R, grid, s);
    if (a.D == 64) return go_rope<float, 64>(R, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace clm

namespace clm {

hipError_t launch_fp8_kv_append(const Fp8AppendArgs& a, hipStream_t s) {
  Fp8AppendP F;
  F.a = AppendP{a.k_new, a.v_new, a.k_cache, a.v_cache, a.block_table, a.len_before,
                a.max_blocks, a.T_new, a.H_kv, a.block_size, a.num_blocks};
  F.k_scale = a.k_scale;
  F.v_scale = a.v_scale;
  F.q = static_cast<uint16_t*>(a.q);
  F.positions = a.positions;
  F.H_q = a.H_q;
  F.G = a.q ? a.H_q / a.H_kv : 0;
  F.log_base = a.q ? log((double)a.rope_base) : 0.0;
  const dim3 grid(a.B * a.H_kv), block(128);
  const bool rope = a.q != nullptr;
  if (a.D == 128 && rope) hipLaunchKernelGGL((fp8_append_kernel<128, true>), grid, block, 0, s, F);
  else if (a.D == 128) hipLaunchKernelGGL((fp8_append_kernel<128, false>), grid, block, 0, s, F);
  else if (a.D == 64 && rope) hipLaunchKernelGGL((fp8_append_kernel<64, true>), grid, block, 0, s, F);
  else if (a.D == 64) hipLaunchKernelGGL((fp8_append_kernel<64, false>), grid, block, 0, s, F);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace clm
