// Device-side helpers shared by the clm kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace clm {

constexpr float kLog2e = 1.4426950408889634f;
// Finite stand-in for -inf as an initial running max: exp2(kNegBig - m) is 0
// for any real score m, and exp2(kNegBig - kNegBig) = 1 multiplies zeros.
constexpr float kNegBig = -1.0e30f;

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// ---- bf16 <-> f32 -----------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two floats to a bf16 pair (lo = a, hi = b), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const f32x2v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---- DPP cross-lane moves within 16-lane rows --------------------------------
// Controls: quad_perm [1,0,3,2] = 0xB1 (xor 1), [2,3,0,1] = 0x4E (xor 2),
// row_half_mirror = 0x141 (lane i <-> 7-i in each half row),
// row_mirror = 0x140 (lane i <-> 15-i in each row).  For sums and maxima these
// act as butterflies: after the four steps every lane of a row holds the
// row-wide result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

template <int LANES>  // 4, 8 or 16 consecutive lanes
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 4 || LANES == 8 || LANES == 16, "group width");
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  if (LANES >= 8) x += dpp_f<0x141>(x);
  if (LANES >= 16) x += dpp_f<0x140>(x);
  return x;
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// ---- whole-wave reductions ------------------------------------------------------
// The four in-row DPP steps give every lane its 16-lane row's result; the four
// rows are then combined from lanes 0, 16, 32 and 48 (readlane), so every lane
// returns the same value and no LDS round trip is made.  Sums add the rows in
// order ((r0 + r1) + r2) + r3.
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  return ((lane_f(x, 0) + lane_f(x, 16)) + lane_f(x, 32)) + lane_f(x, 48);
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return fmaxf(fmaxf(lane_f(x, 0), lane_f(x, 16)), fmaxf(lane_f(x, 32), lane_f(x, 48)));
}
__device__ __forceinline__ int wave_max_i(int x) {
  x = max(x, dpp_i<0xB1>(x));
  x = max(x, dpp_i<0x4E>(x));
  x = max(x, dpp_i<0x141>(x));
  x = max(x, dpp_i<0x140>(x));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
// (value, index) maximum over the wave, ties to the lower index (an order on
// pairs, so the combination order does not matter).  Every lane returns it.
__device__ __forceinline__ void argmax_step(float& bv, int& bi, float ov, int oi) {
  if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
}
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& bv, int& bi) {
  argmax_step(bv, bi, dpp_f<CTRL>(bv), dpp_i<CTRL>(bi));
}
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  argmax_dpp<0xB1>(bv, bi);
  argmax_dpp<0x4E>(bv, bi);
  argmax_dpp<0x141>(bv, bi);
  argmax_dpp<0x140>(bv, bi);
  float v = lane_f(bv, 0);
  int i = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) argmax_step(v, i, lane_f(bv, r), __builtin_amdgcn_readlane(bi, r));
  bv = v;
  bi = i;
}
// Inclusive prefix sum over the 64 lanes (Hillis-Steele, fixed order).
__device__ __forceinline__ float wave_incl_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}
// Integer inclusive prefix sum over the 64 lanes with DPP moves only (no LDS
// round trips): shifts by 1, 2, 4 and 8 inside each 16-lane row, then lane 15
// of rows 0 and 2 is added into rows 1 and 3, and lane 31 into rows 2 and 3.
// Lanes without a source add 0.  Integer addition is exact, so any scan
// order gives the same result.
__device__ __forceinline__ int wave_incl_scan_i(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// ---- global -> LDS DMA -----------------------------------------------------------
// Loads from global memory straight into LDS (no registers): lane l's bytes
// land at lds_byte_addr + 16 l (dma16) or + 4 l (dma4), lds_byte_addr being
// wave-uniform (M0).  The compiler does not see these loads; waits for them
// are explicit s_waitcnt vmcnt(n).  vmcnt retires in issue order, so the
// compiler's own waits stay correct, only more conservative.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "s"(lds_byte_addr) : "memory");
}
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(gptr), "s"(lds_byte_addr) : "memory");
}
// s_waitcnt with only vmcnt = n (0..63) constrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---- streaming loads ----------------------------------------------------------
// Non-temporal global loads (the nt bit): for data streamed once per call
// from HBM (the KV cache).  On gfx950 they sustain a higher HBM read rate
// than default-policy loads on scattered 4 KiB pages.
typedef unsigned nt_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned nt_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_nt(const uint2* p) {
  const nt_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ld_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float4 ld_nt(const float4* p) {
  typedef float f4v __attribute__((ext_vector_type(4)));
  const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

}  // namespace clm
