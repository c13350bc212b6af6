// Kernel-side entry points of libclm.so replaced by stubs, so the host code
// (argument validation, planning, checked-mode plumbing, the decode-loop
// builder) links into a CPU-only executable built with sanitizers.  Every
// stub reports "no device": a call that gets past validation returns
// CLM_ERR_HIP, as it would on a machine without a GPU.
#include <hip/hip_runtime.h>

#include "../../codec_language_model_amd/csrc/clm_launch.h"

namespace clm {
hipError_t launch_kv_append(const AppendArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_rope_kv_append(const RopeAppendArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_fp8_kv_append(const Fp8AppendArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_attention(const AttnArgs&, const AttnPlan&, hipStream_t) { return hipErrorNoDevice; }
hipError_t attention_scratch(void**) { return hipErrorNoDevice; }
hipError_t launch_codebook_head(const HeadArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_sample_or_argmax(const SampleArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_spec_verify(const VerifyArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_advance(int32_t*, int32_t*, int32_t*, const int32_t*, int, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t check_counter(int**) { return hipErrorNoDevice; }
hipError_t launch_check_lengths(const int32_t*, int, int, int, int*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_check_block_table(const int32_t*, const int32_t*, int, int, int, int, int, int*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_check_ints(const int32_t*, int, int, int, int*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_check_uniforms(const float*, int, int*, hipStream_t) { return hipErrorNoDevice; }
}  // namespace clm
