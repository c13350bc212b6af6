// Device-side advance of a decode loop's per-stream state between steps
// (How We Made a Text-to-Speech Model Respond in Sub-50 ms, "Exploiting the
// regular building of the Code Predictor": the whole frame-generation loop
// runs as one graph, so the lengths and positions a step reads must move on
// the device, not from the host).
#include "clm_device.h"
#include "clm_launch.h"

namespace clm {
namespace {

// Stream b advances by num_emitted[b] tokens (speculative verification: the
// accepted drafts plus the residual draw), else by T_new: its length before
// the next append, the visible length of its last query, and the logical
// positions of the next block's T_new tokens.
__global__ __launch_bounds__(256) void advance_kernel(int32_t* len_before, int32_t* kv_len, int32_t* positions,
                                                      const int32_t* num_emitted, int B, int T_new) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int add = num_emitted ? clampi(num_emitted[b], 0, T_new) : T_new;
  len_before[b] += add;
  kv_len[b] += add;
  if (positions)
    for (int t = 0; t < T_new; ++t) positions[(size_t)b * T_new + t] += add;
}

}  // namespace

hipError_t launch_advance(int32_t* len_before, int32_t* kv_len, int32_t* positions, const int32_t* num_emitted,
                          int B, int T_new, hipStream_t s) {
  hipLaunchKernelGGL(advance_kernel, dim3((B + 255) / 256), dim3(256), 0, s, len_before, kv_len, positions,
                     num_emitted, B, T_new);
  return hipGetLastError();
}

}  // namespace clm
