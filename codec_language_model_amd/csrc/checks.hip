// Checked mode (CLM_CHECK=1): validators for device-resident indices.  Each
// adds the number of out-of-range entries it finds to *bad.
#include <mutex>

#include "clm_device.h"
#include "clm_launch.h"

// Checked mode's count of out-of-range entries, in the library's static
// device memory (each GPU holds its own copy).  The name is a host-side
// stand-in; the device address comes from hipGetSymbolAddress, once per
// device (clm::check_counter).
static __device__ __align__(256) int check_count;

namespace clm {
namespace {

__global__ void check_range_kernel(const int32_t* x, int n, int lo, int hi, int* bad) {
  int cnt = 0;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    cnt += (x[i] < lo || x[i] > hi);
  if (cnt) atomicAdd(bad, cnt);
}

__global__ void check_uniform_kernel(const float* u, int n, int* bad) {
  int cnt = 0;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    cnt += !(u[i] >= 0.f && u[i] < 1.f);
  if (cnt) atomicAdd(bad, cnt);
}

// Every block-table entry that covers positions [0, len[b] + len_add) must be
// a valid pool block, and those positions must fit in the row.
__global__ void check_table_kernel(const int32_t* bt, const int32_t* len, int B, int max_blocks,
                                   int len_add, int bs, int num_blocks, int* bad) {
  const int b = blockIdx.x;
  if (b >= B) return;
  const long n = (long)len[b] + len_add;
  if (n < 0 || n > (long)max_blocks * bs) {
    if (threadIdx.x == 0) atomicAdd(bad, 1);
    return;
  }
  const int pages = (int)((n + bs - 1) / bs);
  int cnt = 0;
  for (int p = threadIdx.x; p < pages; p += blockDim.x) {
    const int blk = bt[(size_t)b * max_blocks + p];
    cnt += (blk < 0 || blk >= num_blocks);
  }
  if (cnt) atomicAdd(bad, cnt);
}

int grid_for(int n) {
  int g = (n + 255) / 256;
  return g < 1 ? 1 : (g > 1024 ? 1024 : g);
}

}  // namespace

hipError_t check_counter(int** ptr) {
  constexpr int kMaxDev = 64;
  static int* addr[kMaxDev] = {nullptr};
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_count));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<int*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_check_lengths(const int32_t* len, int n, int lo, int hi, int* bad, hipStream_t s) {
  hipLaunchKernelGGL(check_range_kernel, dim3(grid_for(n)), dim3(256), 0, s, len, n, lo, hi, bad);
  return hipGetLastError();
}

hipError_t launch_check_ints(const int32_t* x, int n, int lo, int hi, int* bad, hipStream_t s) {
  return launch_check_lengths(x, n, lo, hi, bad, s);
}

hipError_t launch_check_uniforms(const float* u, int n, int* bad, hipStream_t s) {
  hipLaunchKernelGGL(check_uniform_kernel, dim3(grid_for(n)), dim3(256), 0, s, u, n, bad);
  return hipGetLastError();
}

hipError_t launch_check_block_table(const int32_t* bt, const int32_t* len, int B, int max_blocks,
                                    int len_add, int block_size, int num_blocks, int* bad,
                                    hipStream_t s) {
  hipLaunchKernelGGL(check_table_kernel, dim3(B), dim3(256), 0, s, bt, len, B, max_blocks, len_add,
                     block_size, num_blocks, bad);
  return hipGetLastError();
}

}  // namespace clm
