// Multi-step decode loop captured as one HIP graph (How We Made a
// Text-to-Speech Model Respond in Sub-50 ms, "Exploiting the regular building
// of the Code Predictor": the frame-generation loop as a single graph;
// section "Additional serving optimizations": graphs kept per batch size).
// The loop is built from the C-ABI calls themselves - each only enqueues
// kernels on its stream, so recording them on a capture stream gives the same
// kernels, arguments and results as eager calls - plus the device-side
// advance of the lengths and positions between steps.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <new>
#include <type_traits>
#include <vector>

#include "../../include/clm.h"
#include "clm_launch.h"

struct clm_decode_loop {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int n_steps = 0;
};

namespace {

size_t elem_bytes(clm_dtype dt) { return dt == CLM_BF16 ? 2 : 4; }

template <class T>
T* step_ptr(T* base, int s, size_t step_bytes) {
  if (!base) return nullptr;
  using B = typename std::conditional<std::is_const<T>::value, const char, char>::type;
  return reinterpret_cast<T*>(reinterpret_cast<B*>(base) + (size_t)s * step_bytes);
}

// Enqueues step s of the loop on `st`.
int record_step(const clm_decode_step_desc& d, int s, hipStream_t st) {
  const size_t e = elem_bytes(d.dt);
  const int M = d.B * d.Kq;
  const size_t kv_step = (size_t)d.B * d.Kq * d.H_kv * d.D * e;
  const size_t q_step = (size_t)d.B * d.Kq * d.H_q * d.D * e;
  void* q = step_ptr(d.q, s, q_step);
  const void* kn = step_ptr(d.k_new, s, kv_step);
  const void* vn = step_ptr(d.v_new, s, kv_step);
  const bool f8 = d.k_scale != nullptr;
  int rc;
  if (f8 && d.positions)
    rc = clm_rope_kv_cache_append_fp8(q, kn, vn, d.k_cache, d.v_cache, d.k_scale, d.v_scale, d.block_table,
                                      d.max_blocks, d.len_before, d.positions, d.rope_base, d.B, d.Kq, d.H_q,
                                      d.H_kv, d.D, d.block_size, d.num_blocks, st);
  else if (f8)
    rc = clm_kv_cache_append_fp8(kn, vn, d.k_cache, d.v_cache, d.k_scale, d.v_scale, d.block_table, d.max_blocks,
                                 d.len_before, d.B, d.Kq, d.H_kv, d.D, d.block_size, d.num_blocks, st);
  else if (d.positions)
    rc = clm_rope_kv_cache_append(q, kn, vn, d.k_cache, d.v_cache, d.block_table, d.max_blocks, d.len_before,
                                  d.positions, d.rope_base, d.B, d.Kq, d.H_q, d.H_kv, d.D, d.block_size,
                                  d.num_blocks, d.dt, st);
  else
    rc = clm_kv_cache_append(kn, vn, d.k_cache, d.v_cache, d.block_table, d.max_blocks, d.len_before, d.B, d.Kq,
                             d.H_kv, d.D, d.block_size, d.num_blocks, d.dt, st);
  if (rc != CLM_OK) return rc;
  void* o = step_ptr(d.o, s, q_step);
  const float scale = 1.0f / __builtin_sqrtf((float)d.D);
  if (f8)
    rc = clm_decode_attention_fp8(q, d.k_cache, d.v_cache, d.k_scale, d.v_scale, d.block_table, d.max_blocks,
                                  d.kv_len, d.max_kv_len, o, d.B, d.Kq, d.H_q, d.H_kv, d.D, d.block_size,
                                  d.num_blocks, scale, d.attn_workspace, d.attn_workspace_bytes, st);
  else if (d.attn_workspace)
    rc = clm_decode_attention(q, d.k_cache, d.v_cache, d.block_table, d.max_blocks, d.kv_len, d.max_kv_len, o, d.B,
                              d.Kq, d.H_q, d.H_kv, d.D, d.block_size, d.num_blocks, scale, d.dt, d.attn_workspace,
                              d.attn_workspace_bytes, st);
  else
    rc = clm_decode_attention_noalloc(q, d.k_cache, d.v_cache, d.block_table, d.max_blocks, d.kv_len,
                                      d.max_kv_len, o, d.B, d.Kq, d.H_q, d.H_kv, d.D, d.block_size, d.num_blocks,
                                      scale, d.dt, st);
  if (rc != CLM_OK) return rc;
  float* logits = step_ptr(d.logits, s, (size_t)M * d.V * sizeof(float));
  rc = d.W2 ? clm_codebook_head_mlp(o, d.W, d.W2, d.G, d.head_id, d.act, logits, M, d.H_q * d.D, d.F, d.V, d.dt,
                                     nullptr, 0, st)
            : clm_codebook_head(o, d.W, d.G, d.head_id, logits, M, d.H_q * d.D, d.V, d.dt, nullptr, 0, st);
  if (rc != CLM_OK) return rc;
  const int32_t* emitted = nullptr;
  if (d.mode == 2 || d.mode == 3) {
    // mode 3: the Kq target rows score the last kept token and Kd = Kq - 1 drafts
    const int Kd = d.mode == 3 ? d.Kq - 1 : d.Kq;
    const size_t Md = (size_t)d.B * Kd;
    int32_t* num = step_ptr(d.num_emitted, s, (size_t)d.B * sizeof(int32_t));
    const float* dp = step_ptr(d.draft_probs, s, Md * d.V * sizeof(float));
    const int32_t* dtok = step_ptr(d.draft_tokens, s, Md * sizeof(int32_t));
    const float* ua = step_ptr(d.u_accept, s, Md * sizeof(float));
    const float* ur = step_ptr(d.u_resample, s, (size_t)d.B * sizeof(float));
    int32_t* ot = step_ptr(d.out_tokens, s, (size_t)M * sizeof(int32_t));
    rc = d.mode == 3 ? clm_spec_verify_bonus(logits, dp, dtok, ua, ur, d.spec_temperature, d.B, Kd, d.V, ot, num, st)
                     : clm_spec_verify(logits, dp, dtok, ua, ur, d.spec_temperature, d.B, Kd, d.V, ot, num, st);
    emitted = num;
  } else {
    rc = clm_sample_or_argmax(logits, M, d.V, d.V,
                              d.mode == 1 ? step_ptr(d.temperature, s, (size_t)M * sizeof(float)) : nullptr,
                              d.mode == 1 ? step_ptr(d.uniforms, s, (size_t)M * sizeof(float)) : nullptr,
                              nullptr, step_ptr(d.tokens, s, (size_t)M * sizeof(int32_t)), st);
  }
  if (rc != CLM_OK) return rc;
  return clm_advance_lengths(d.len_before, d.kv_len, d.positions, emitted, d.B, d.Kq, st);
}

int check_desc(const clm_decode_step_desc& d) {
  if (!d.k_cache || !d.v_cache || !d.block_table || !d.len_before || !d.kv_len || !d.k_new || !d.v_new || !d.q ||
      !d.W || !d.o || !d.logits)
    return CLM_ERR_INVALID_ARG;
  if (d.B < 1 || d.Kq < 1 || d.H_q < 1 || d.H_kv < 1 || d.D < 1 || d.G < 1 || d.V < 1) return CLM_ERR_INVALID_ARG;
  if (d.mode == 0 || d.mode == 1) {
    if (!d.tokens) return CLM_ERR_INVALID_ARG;
    if (d.mode == 1 && (!d.temperature || !d.uniforms)) return CLM_ERR_INVALID_ARG;
  } else if (d.mode == 2 || d.mode == 3) {
    if (!d.draft_probs || !d.draft_tokens || !d.u_accept || !d.u_resample || !d.out_tokens || !d.num_emitted)
      return CLM_ERR_INVALID_ARG;
    if (d.mode == 3 && d.Kq < 2) return CLM_ERR_INVALID_ARG;
  } else {
    return CLM_ERR_INVALID_ARG;
  }
  if (!d.k_scale != !d.v_scale) return CLM_ERR_INVALID_ARG;
  if (d.W2 && (!d.act || d.F < 1)) return CLM_ERR_INVALID_ARG;
  if (d.W2 && d.dt != CLM_BF16) return CLM_ERR_UNSUPPORTED;
  if (d.k_scale && (d.dt != CLM_BF16 || !d.attn_workspace)) return CLM_ERR_UNSUPPORTED;
  return CLM_OK;
}

}  // namespace

extern "C" {

int clm_advance_lengths(int32_t* len_before, int32_t* kv_len, int32_t* positions, const int32_t* num_emitted,
                        int B, int T_new, hipStream_t stream) {
  if (!len_before || !kv_len || B < 1 || T_new < 1) return CLM_ERR_INVALID_ARG;
  return clm::launch_advance(len_before, kv_len, positions, num_emitted, B, T_new, stream) == hipSuccess
             ? CLM_OK : CLM_ERR_HIP;
}

int clm_pick_bucket(const int32_t* bucket_sizes, int n, int B) {
  if (!bucket_sizes || n < 1 || B < 1) return -1;
  int best = -1;
  for (int i = 0; i < n; ++i)
    if (bucket_sizes[i] >= B && (best < 0 || bucket_sizes[i] < bucket_sizes[best])) best = i;
  return best;
}

int clm_decode_loop_create(const clm_decode_step_desc* desc, int n_steps, clm_decode_loop** loop) {
  if (!desc || !loop || n_steps < 1 || n_steps > 1024) return CLM_ERR_INVALID_ARG;
  *loop = nullptr;
  const clm_decode_step_desc d = *desc;
  int rc = check_desc(d);
  if (rc != CLM_OK) return rc;
  if (clm::checked_mode()) return CLM_ERR_UNSUPPORTED;
  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return CLM_ERR_HIP;
  hipGraph_t graph = nullptr;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return CLM_ERR_HIP;
  }
  for (int s = 0; s < n_steps && rc == CLM_OK; ++s) rc = record_step(d, s, cs);
  const hipError_t ec = hipStreamEndCapture(cs, &graph);
  (void)hipStreamDestroy(cs);
  if (rc == CLM_OK && ec != hipSuccess) rc = CLM_ERR_HIP;
  if (rc != CLM_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return rc;
  }
  hipGraphExec_t exec = nullptr;
  if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return CLM_ERR_HIP;
  }
  clm_decode_loop* l = new (std::nothrow) clm_decode_loop;
  if (!l) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return CLM_ERR_HIP;
  }
  l->graph = graph;
  l->exec = exec;
  l->n_steps = n_steps;
  *loop = l;
  return CLM_OK;
}

int clm_decode_loop_launch(clm_decode_loop* loop, hipStream_t stream) {
  if (!loop || !loop->exec) return CLM_ERR_INVALID_ARG;
  return hipGraphLaunch(loop->exec, stream) == hipSuccess ? CLM_OK : CLM_ERR_HIP;
}

int clm_decode_loop_destroy(clm_decode_loop* loop) {
  if (!loop) return CLM_ERR_INVALID_ARG;
  int rc = CLM_OK;
  if (loop->exec && hipGraphExecDestroy(loop->exec) != hipSuccess) rc = CLM_ERR_HIP;
  if (loop->graph && hipGraphDestroy(loop->graph) != hipSuccess) rc = CLM_ERR_HIP;
  delete loop;
  return rc;
}

}  // extern "C"
