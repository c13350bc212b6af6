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

  for (int e = threadIdx.x; e < P.T_new * CH; e += blockDim.x) {
    const int t = e / CH, ch = e - (e / CH) * CH;
    const int pos = lb + t;
    if (pos < 0) continue;
    const int page = pos / P.bs;
    if (page >= P.max_blocks) continue;
    const int blk = bt_row[page];
    if (blk < 0 || blk >= P.num_blocks) continue;
    const int slot = pos - page * P.bs;
    const T* src = kn + ((size_t)(b * P.T_new + t) * P.H_kv + h) * D + ch * VE;
    T* dst = kc + (((size_t)blk * P.H_kv + h) * P.bs + slot) * D + ch * VE;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  }
  for (int e = threadIdx.x; e < P.T_new * D; e += blockDim.x) {
    const int t = e / D, d = e - (e / D) * D;
    const int pos = lb + t;
    if (pos < 0) continue;
    const int page = pos / P.bs;
    if (page >= P.max_blocks) continue;
    const int blk = bt_row[page];
    if (blk < 0 || blk >= P.num_blocks) continue;
    const int slot = pos - page * P.bs;
    vc[(((size_t)blk * P.H_kv + h) * D + d) * P.bs + slot] =
        vn[((size_t)(b * P.T_new + t) * P.H_kv + h) * D + d];
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
