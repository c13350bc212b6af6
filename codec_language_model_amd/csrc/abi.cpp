// C ABI of libclm.so: argument validation, checked mode, kernel dispatch.
// Every function validates host-visible arguments before its first HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <atomic>
#include <cstring>

#include "../../include/clm.h"
#include "clm_launch.h"

namespace {

bool env_checked() {
  const char* v = std::getenv("CLM_CHECK");
  return v && *v && std::strcmp(v, "0") != 0;
}
// Checked mode: CLM_CHECK at load time, then clm_set_checked.
std::atomic<int> g_checked_flag{env_checked() ? 1 : 0};
inline bool checked() { return g_checked_flag.load(std::memory_order_relaxed) != 0; }

// (stream, KV head) pairs one attention call takes.
constexpr long kMaxStreamHeads = 65536;


bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool dt_ok(clm_dtype dt) { return dt == CLM_F32 || dt == CLM_BF16; }
bool bs_ok(int bs) { return bs >= 16 && bs <= 256 && bs % 16 == 0; }

// Runs `launch(bad)` (validators on `stream`), waits, and reports whether any
// device value was out of range.
// The count lives in the library's static device memory (clm::check_counter),
// so checked mode allocates nothing.
template <class F>
int run_checks(hipStream_t stream, F launch) {
  int* bad = nullptr;
  if (clm::check_counter(&bad) != hipSuccess) return CLM_ERR_HIP;
  if (hipMemsetAsync(bad, 0, sizeof(int), stream) != hipSuccess) return CLM_ERR_HIP;
  if (launch(bad) != hipSuccess) return CLM_ERR_HIP;
  int h = 0;
  if (hipStreamSynchronize(stream) != hipSuccess) return CLM_ERR_HIP;
  if (hipMemcpy(&h, bad, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess) return CLM_ERR_HIP;
  return h ? CLM_ERR_DEVICE_DATA : CLM_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? CLM_OK : CLM_ERR_HIP; }

}  // namespace

namespace clm {
bool checked_mode() { return checked(); }
}  // namespace clm

extern "C" {

const char* clm_status_string(int status) {
  switch (status) {
    case CLM_OK: return "CLM_OK";
    case CLM_ERR_INVALID_ARG: return "CLM_ERR_INVALID_ARG";
    case CLM_ERR_UNSUPPORTED: return "CLM_ERR_UNSUPPORTED";
    case CLM_ERR_CAPACITY: return "CLM_ERR_CAPACITY";
    case CLM_ERR_WORKSPACE: return "CLM_ERR_WORKSPACE";
    case CLM_ERR_HIP: return "CLM_ERR_HIP";
    case CLM_ERR_DEVICE_DATA: return "CLM_ERR_DEVICE_DATA";
  }
  return "CLM_ERR_UNKNOWN";
}

int clm_version(void) { return 300; }

int clm_set_checked(int on) { return g_checked_flag.exchange(on ? 1 : 0) ; }

int clm_kv_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int32_t* block_table, int max_blocks, const int32_t* len_before,
                        int B, int T_new, int H_kv, int D, int block_size, int num_blocks,
                        clm_dtype dt, hipStream_t stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !len_before) return CLM_ERR_INVALID_ARG;
  if (B < 1 || T_new < 1 || H_kv < 1 || D < 1 || max_blocks < 1 || num_blocks < 1 || block_size < 1)
    return CLM_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(k_cache, 16)) return CLM_ERR_INVALID_ARG;
  if (!dt_ok(dt) || (D != 64 && D != 128) || !bs_ok(block_size)) return CLM_ERR_UNSUPPORTED;
  if ((long)T_new > (long)max_blocks * block_size) return CLM_ERR_CAPACITY;
  if ((long)B * H_kv > (1L << 31) - 1) return CLM_ERR_UNSUPPORTED;
  if (checked()) {
    const long lim = (long)max_blocks * block_size - T_new;
    int st = run_checks(stream, [&](int* bad) {
      hipError_t e = clm::launch_check_lengths(len_before, B, 0, (int)(lim > 0x7fffffff ? 0x7fffffff : lim), bad, stream);
      if (e != hipSuccess) return e;
      return clm::launch_check_block_table(block_table, len_before, B, max_blocks, T_new, block_size,
                                           num_blocks, bad, stream);
    });
    if (st != CLM_OK) return st;
  }
  clm::AppendArgs a{k_new, v_new, k_cache, v_cache, block_table, len_before,
                    max_blocks, B, T_new, H_kv, D, block_size, num_blocks, dt == CLM_BF16};
  return hip_status(clm::launch_kv_append(a, stream));
}

int clm_rope_kv_cache_append(void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* block_table, int max_blocks, const int32_t* len_before,
                             const int32_t* positions, float rope_base, int B, int T_new, int H_q,
                             int H_kv, int D, int block_size, int num_blocks, clm_dtype dt,
                             hipStream_t stream) {
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !block_table || !len_before || !positions)
    return CLM_ERR_INVALID_ARG;
  if (B < 1 || T_new < 1 || H_q < 1 || H_kv < 1 || D < 1 || max_blocks < 1 || num_blocks < 1 ||
      block_size < 1 || H_q % H_kv != 0)
    return CLM_ERR_INVALID_ARG;
  if (!std::isfinite(rope_base) || !(rope_base > 1.f)) return CLM_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(k_cache, 16)) return CLM_ERR_INVALID_ARG;
  if (!dt_ok(dt) || (D != 64 && D != 128) || !bs_ok(block_size)) return CLM_ERR_UNSUPPORTED;
  if ((long)T_new > (long)max_blocks * block_size) return CLM_ERR_CAPACITY;
  if ((long)B * H_kv > (1L << 31) - 1) return CLM_ERR_UNSUPPORTED;
  if (checked()) {
    const long lim = (long)max_blocks * block_size - T_new;
    int st = run_checks(stream, [&](int* bad) {
      hipError_t e = clm::launch_check_lengths(len_before, B, 0, (int)(lim > 0x7fffffff ? 0x7fffffff : lim), bad, stream);
      if (e != hipSuccess) return e;
      return clm::launch_check_block_table(block_table, len_before, B, max_blocks, T_new, block_size,
                                           num_blocks, bad, stream);
    });
    if (st != CLM_OK) return st;
  }
  clm::RopeAppendArgs a{q, k_new, v_new, k_cache, v_cache, block_table, max_blocks, len_before, positions,
                        rope_base, B, T_new, H_q, H_kv, D, block_size, num_blocks, dt == CLM_BF16};
  return hip_status(clm::launch_rope_kv_append(a, stream));
}

size_t clm_decode_attention_workspace_size(int B, int Kq, int H_q, int H_kv, int D, int max_kv_len) {
  if (B < 1 || Kq < 1 || H_q < 1 || H_kv < 1 || (D != 64 && D != 128) || max_kv_len < Kq) return 0;
  if (H_q % H_kv != 0 || B > 4096 || (long)B * H_kv > kMaxStreamHeads) return 0;
  clm::AttnPlan p;
  if (!clm::plan_decode_attention(B, Kq, H_q, H_kv, D, max_kv_len, &p)) return 0;
  return p.total_bytes;
}

int clm_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, int max_blocks, const int32_t* kv_len,
                         int max_kv_len, void* o, int B, int Kq, int H_q, int H_kv, int D,
                         int block_size, int num_blocks, float scale, clm_dtype dt,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !block_table || !kv_len || !o) return CLM_ERR_INVALID_ARG;
  if (B < 1 || Kq < 1 || H_q < 1 || H_kv < 1 || D < 1 || max_blocks < 1 || num_blocks < 1 ||
      block_size < 1)
    return CLM_ERR_INVALID_ARG;
  if (H_q % H_kv != 0 || max_kv_len < Kq || !std::isfinite(scale)) return CLM_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16)) return CLM_ERR_INVALID_ARG;
  if (!dt_ok(dt) || (D != 64 && D != 128) || !bs_ok(block_size) || B > 4096) return CLM_ERR_UNSUPPORTED;
  if ((long)B * H_kv > kMaxStreamHeads) return CLM_ERR_UNSUPPORTED;
  if ((H_q / H_kv) * Kq > 16) return CLM_ERR_UNSUPPORTED;
  clm::AttnPlan p;
  if (!clm::plan_decode_attention(B, Kq, H_q, H_kv, D, max_kv_len, &p)) return CLM_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.total_bytes || !aligned(workspace, 256)) return CLM_ERR_WORKSPACE;
  if (checked()) {
    const long cap = (long)max_blocks * block_size;
    const int hi = (int)(cap < max_kv_len ? cap : max_kv_len);
    int st = run_checks(stream, [&](int* bad) {
      hipError_t e = clm::launch_check_lengths(kv_len, B, Kq, hi, bad, stream);
      if (e != hipSuccess) return e;
      return clm::launch_check_block_table(block_table, kv_len, B, max_blocks, 0, block_size,
                                           num_blocks, bad, stream);
    });
    if (st != CLM_OK) return st;
  }
  clm::AttnArgs a{q, k_cache, v_cache, block_table, kv_len, o, workspace, max_blocks, max_kv_len,
                  B, Kq, H_q, H_kv, D, block_size, num_blocks, scale, dt == CLM_BF16};
  return hip_status(clm::launch_decode_attention(a, p, stream));
}

int clm_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, int max_blocks, const int32_t* kv_len,
                                 int max_kv_len, void* o, int B, int Kq, int H_q, int H_kv, int D,
                                 int block_size, int num_blocks, float scale, clm_dtype dt,
                                 hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !block_table || !kv_len || !o) return CLM_ERR_INVALID_ARG;
  if (B < 1 || Kq < 1 || H_q < 1 || H_kv < 1 || D < 1 || max_blocks < 1 || num_blocks < 1 ||
      block_size < 1)
    return CLM_ERR_INVALID_ARG;
  if (H_q % H_kv != 0 || max_kv_len < Kq || !std::isfinite(scale)) return CLM_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16)) return CLM_ERR_INVALID_ARG;
  if (!dt_ok(dt) || (D != 64 && D != 128) || !bs_ok(block_size) || B > 4096) return CLM_ERR_UNSUPPORTED;
  if ((long)B * H_kv > kMaxStreamHeads) return CLM_ERR_UNSUPPORTED;
  if ((H_q / H_kv) * Kq > 16) return CLM_ERR_UNSUPPORTED;
  clm::AttnPlan p;
  if (!clm::plan_decode_attention(B, Kq, H_q, H_kv, D, max_kv_len, &p)) return CLM_ERR_UNSUPPORTED;
  if (p.total_bytes > clm::kAttentionScratchBytes) return CLM_ERR_WORKSPACE;
  void* scratch = nullptr;
  if (clm::attention_scratch(&scratch) != hipSuccess) return CLM_ERR_HIP;
  if (checked()) {
    const long cap = (long)max_blocks * block_size;
    const int hi = (int)(cap < max_kv_len ? cap : max_kv_len);
    int st = run_checks(stream, [&](int* bad) {
      hipError_t e = clm::launch_check_lengths(kv_len, B, Kq, hi, bad, stream);
      if (e != hipSuccess) return e;
      return clm::launch_check_block_table(block_table, kv_len, B, max_blocks, 0, block_size,
                                           num_blocks, bad, stream);
    });
    if (st != CLM_OK) return st;
  }
  clm::AttnArgs a{q, k_cache, v_cache, block_table, kv_len, o, scratch, max_blocks, max_kv_len,
                  B, Kq, H_q, H_kv, D, block_size, num_blocks, scale, dt == CLM_BF16};
  return hip_status(clm::launch_decode_attention(a, p, stream));
}

int clm_kv_cache_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            float* k_scale, float* v_scale, const int32_t* block_table, int max_blocks,
                            const int32_t* len_before, int B, int T_new, int H_kv, int D, int block_size,
                            int num_blocks, hipStream_t stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !k_scale || !v_scale || !block_table || !len_before)
    return CLM_ERR_INVALID_ARG;
  if (B < 1 || T_new < 1 || H_kv < 1 || D < 1 || max_blocks < 1 || num_blocks < 1 || block_size < 1)
    return CLM_ERR_INVALID_ARG;
  if ((D != 64 && D != 128) || !bs_ok(block_size)) return CLM_ERR_UNSUPPORTED;
  if ((long)T_new > (long)max_blocks * block_size) return CLM_ERR_CAPACITY;
  if ((long)B * H_kv > (1L << 31) - 1) return CLM_ERR_UNSUPPORTED;
  if (checked()) {
    const long lim = (long)max_blocks * block_size - T_new;
    int st = run_checks(stream, [&](int* bad) {
      hipError_t e = clm::launch_check_lengths(len_before, B, 0, (int)(lim > 0x7fffffff ? 0x7fffffff : lim), bad, stream);
      if (e != hipSuccess) return e;
      return clm::launch_check_block_table(block_table, len_before, B, max_blocks, T_new, block_size,
                                           num_blocks, bad, stream);
    });
    if (st != CLM_OK) return st;
  }
  clm::Fp8AppendArgs a{k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, len_before,
                       max_blocks, B, T_new, H_kv, D, block_size, num_blocks};
  return hip_status(clm::launch_fp8_kv_append(a, stream));
}

int clm_rope_kv_cache_append_fp8(void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 float* k_scale, float* v_scale, const int32_t* block_table, int max_blocks,
                                 const int32_t* len_before, const int32_t* positions, float rope_base, int B,
                                 int T_new, int H_q, int H_kv, int D, int block_size, int num_blocks,
                                 hipStream_t stream) {
  if (!q || !positions) return CLM_ERR_INVALID_ARG;
  if (H_q < 1 || H_kv < 1 || H_q % H_kv != 0) return CLM_ERR_INVALID_ARG;
  if (!std::isfinite(rope_base) || !(rope_base > 1.f)) return CLM_ERR_INVALID_ARG;
  if (!aligned(q, 16)) return CLM_ERR_INVALID_ARG;
  if (!k_new || !v_new || !k_cache || !v_cache || !k_scale || !v_scale || !block_table || !len_before)
    return CLM_ERR_INVALID_ARG;
  if (B < 1 || T_new < 1 || D < 1 || max_blocks < 1 || num_blocks < 1 || block_size < 1)
    return CLM_ERR_INVALID_ARG;
  if ((D != 64 && D != 128) || !bs_ok(block_size)) return CLM_ERR_UNSUPPORTED;
  if ((long)T_new > (long)max_blocks * block_size) return CLM_ERR_CAPACITY;
  if ((long)B * H_kv > (1L << 31) - 1) return CLM_ERR_UNSUPPORTED;
  if (checked()) {
    const long lim = (long)max_blocks * block_size - T_new;
    int st = run_checks(stream, [&](int* bad) {
      hipError_t e = clm::launch_check_lengths(len_before, B, 0, (int)(lim > 0x7fffffff ? 0x7fffffff : lim), bad, stream);
      if (e != hipSuccess) return e;
      return clm::launch_check_block_table(block_table, len_before, B, max_blocks, T_new, block_size,
                                           num_blocks, bad, stream);
    });
    if (st != CLM_OK) return st;
  }
  clm::Fp8AppendArgs a{k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, len_before,
                       max_blocks, B, T_new, H_kv, D, block_size, num_blocks};
  a.q = q;
  a.positions = positions;
  a.rope_base = rope_base;
  a.H_q = H_q;
  return hip_status(clm::launch_fp8_kv_append(a, stream));
}

int clm_decode_attention_fp8(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                             const float* v_scale, const int32_t* block_table, int max_blocks,
                             const int32_t* kv_len, int max_kv_len, void* o, int B, int Kq, int H_q, int H_kv,
                             int D, int block_size, int num_blocks, float scale, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !block_table || !kv_len || !o)
    return CLM_ERR_INVALID_ARG;
  if (B < 1 || Kq < 1 || H_q < 1 || H_kv < 1 || D < 1 || max_blocks < 1 || num_blocks < 1 ||
      block_size < 1)
    return CLM_ERR_INVALID_ARG;
  if (H_q % H_kv != 0 || max_kv_len < Kq || !std::isfinite(scale)) return CLM_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_scale, 16) ||
      !aligned(v_scale, 16))
    return CLM_ERR_INVALID_ARG;
  if ((D != 64 && D != 128) || !bs_ok(block_size) || B > 4096) return CLM_ERR_UNSUPPORTED;
  if ((long)B * H_kv > kMaxStreamHeads) return CLM_ERR_UNSUPPORTED;
  if ((H_q / H_kv) * Kq > 16) return CLM_ERR_UNSUPPORTED;
  clm::AttnPlan p;
  if (!clm::plan_decode_attention(B, Kq, H_q, H_kv, D, max_kv_len, &p)) return CLM_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.total_bytes || !aligned(workspace, 256)) return CLM_ERR_WORKSPACE;
  if (checked()) {
    const long cap = (long)max_blocks * block_size;
    const int hi = (int)(cap < max_kv_len ? cap : max_kv_len);
    int st = run_checks(stream, [&](int* bad) {
      hipError_t e = clm::launch_check_lengths(kv_len, B, Kq, hi, bad, stream);
      if (e != hipSuccess) return e;
      return clm::launch_check_block_table(block_table, kv_len, B, max_blocks, 0, block_size,
                                           num_blocks, bad, stream);
    });
    if (st != CLM_OK) return st;
  }
  clm::AttnArgs a{q, k_cache, v_cache, block_table, kv_len, o, workspace, max_blocks, max_kv_len,
                  B, Kq, H_q, H_kv, D, block_size, num_blocks, scale, true, k_scale, v_scale};
  return hip_status(clm::launch_decode_attention(a, p, stream));
}

size_t clm_codebook_head_workspace_size(int M, int d, int V, int G, clm_dtype dt) {
  if (M < 1 || d < 1 || V < 1 || G < 1 || G > 8 || M > 65536 || !dt_ok(dt)) return 0;
  if (dt != CLM_BF16) return 0;
  return clm::plan_codebook_head(M, V, G).workspace_bytes;
}

size_t clm_codebook_head_mlp_workspace_size(int M, int d, int F, int V, int G) {
  if (M < 1 || d < 1 || F < 1 || V < 1 || G < 1 || G > 8 || M > 65536) return 0;
  const size_t a = clm::plan_codebook_head(M, F, G).workspace_bytes;
  const size_t b = clm::plan_codebook_head(M, V, G).workspace_bytes;
  return a > b ? a : b;
}

static bool workspace_ok(const void* ws, size_t bytes, size_t need) {
  if (ws && !aligned(ws, 256)) return false;
  if (need == 0) return true;
  return ws && bytes >= need;
}

int clm_codebook_head(const void* h, const void* const* W, int G, const int32_t* head_id,
                      float* logits, int M, int d, int V, clm_dtype dt, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  if (!h || !W || !logits) return CLM_ERR_INVALID_ARG;
  if (M < 1 || d < 1 || V < 1 || G < 1 || G > 8) return CLM_ERR_INVALID_ARG;
  if (G > 1 && !head_id) return CLM_ERR_INVALID_ARG;
  for (int g = 0; g < G; ++g)
    if (!W[g] || !aligned(W[g], 16)) return CLM_ERR_INVALID_ARG;
  if (!aligned(h, 16)) return CLM_ERR_INVALID_ARG;
  if (!dt_ok(dt) || M > 65536) return CLM_ERR_UNSUPPORTED;
  if (dt == CLM_BF16 && d % 128 != 0) return CLM_ERR_UNSUPPORTED;
  if (dt == CLM_F32 && d % 4 != 0) return CLM_ERR_UNSUPPORTED;
  if (!workspace_ok(workspace, workspace_bytes, clm_codebook_head_workspace_size(M, d, V, G, dt)))
    return CLM_ERR_WORKSPACE;
  if (checked() && G > 1) {
    int st = run_checks(stream, [&](int* bad) { return clm::launch_check_ints(head_id, M, 0, G - 1, bad, stream); });
    if (st != CLM_OK) return st;
  }
  clm::HeadArgs a;
  a.h = h;
  for (int g = 0; g < 8; ++g) a.W[g] = g < G ? W[g] : W[0];
  a.G = G; a.head_id = head_id; a.logits = logits; a.M = M; a.d = d; a.V = V;
  a.bf16 = dt == CLM_BF16;
  a.act = nullptr;
  return hip_status(clm::launch_codebook_head(a, stream));
}

int clm_codebook_head_mlp(const void* h, const void* const* W1, const void* const* W2, int G,
                          const int32_t* head_id, void* act, float* logits, int M, int d, int F, int V,
                          clm_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!h || !W1 || !W2 || !act || !logits) return CLM_ERR_INVALID_ARG;
  if (M < 1 || d < 1 || F < 1 || V < 1 || G < 1 || G > 8) return CLM_ERR_INVALID_ARG;
  if (G > 1 && !head_id) return CLM_ERR_INVALID_ARG;
  for (int g = 0; g < G; ++g)
    if (!W1[g] || !W2[g] || !aligned(W1[g], 16) || !aligned(W2[g], 16)) return CLM_ERR_INVALID_ARG;
  if (!aligned(h, 16) || !aligned(act, 16)) return CLM_ERR_INVALID_ARG;
  if (dt != CLM_BF16) return CLM_ERR_UNSUPPORTED;
  if (M > 65536 || d % 128 != 0 || F % 128 != 0) return CLM_ERR_UNSUPPORTED;
  if (!workspace_ok(workspace, workspace_bytes, clm_codebook_head_mlp_workspace_size(M, d, F, V, G)))
    return CLM_ERR_WORKSPACE;
  if (checked() && G > 1) {
    int st = run_checks(stream, [&](int* bad) { return clm::launch_check_ints(head_id, M, 0, G - 1, bad, stream); });
    if (st != CLM_OK) return st;
  }
  clm::HeadArgs a;
  a.h = h;
  for (int g = 0; g < 8; ++g) a.W[g] = g < G ? W1[g] : W1[0];
  a.G = G; a.head_id = head_id; a.logits = nullptr; a.M = M; a.d = d; a.V = F;
  a.bf16 = true;
  a.act = static_cast<uint16_t*>(act);
  hipError_t e = clm::launch_codebook_head(a, stream);
  if (e != hipSuccess) return hip_status(e);
  a.h = act;
  for (int g = 0; g < 8; ++g) a.W[g] = g < G ? W2[g] : W2[0];
  a.logits = logits; a.d = F; a.V = V; a.act = nullptr;
  return hip_status(clm::launch_codebook_head(a, stream));
}

int clm_sample_or_argmax(const float* logits, int M, int V, int ld, const float* temperature,
                         const float* uniforms, const int32_t* vocab_valid, int32_t* tokens,
                         hipStream_t stream) {
  if (!logits || !tokens || M < 1 || V < 1 || ld < V) return CLM_ERR_INVALID_ARG;
  if (temperature && !uniforms) return CLM_ERR_INVALID_ARG;
  if (V > (1 << 20)) return CLM_ERR_UNSUPPORTED;
  if (checked()) {
    int st = run_checks(stream, [&](int* bad) {
      hipError_t e = hipSuccess;
      if (vocab_valid) e = clm::launch_check_ints(vocab_valid, M, 1, V, bad, stream);
      if (e == hipSuccess && uniforms && temperature) e = clm::launch_check_uniforms(uniforms, M, bad, stream);
      return e;
    });
    if (st != CLM_OK) return st;
  }
  clm::SampleArgs a{logits, M, V, ld, temperature, uniforms, vocab_valid, tokens};
  return hip_status(clm::launch_sample_or_argmax(a, stream));
}

static int spec_verify_impl(const float* target_logits, const float* draft_probs,
                            const int32_t* draft_tokens, const float* u_accept, const float* u_resample,
                            float temperature, int B, int K, int V, int32_t* out_tokens,
                            int32_t* num_emitted, int bonus, hipStream_t stream) {
  if (!target_logits || !draft_probs || !draft_tokens || !u_accept || !u_resample || !out_tokens ||
      !num_emitted)
    return CLM_ERR_INVALID_ARG;
  if (B < 1 || K < 1 || V < 1 || !std::isfinite(temperature) || temperature < 0.f) return CLM_ERR_INVALID_ARG;
  if (K + bonus > 16 || V > (1 << 20)) return CLM_ERR_UNSUPPORTED;
  if (checked()) {
    int st = run_checks(stream, [&](int* bad) {
      hipError_t e = clm::launch_check_ints(draft_tokens, B * K, 0, V - 1, bad, stream);
      if (e == hipSuccess) e = clm::launch_check_uniforms(u_accept, B * K, bad, stream);
      if (e == hipSuccess) e = clm::launch_check_uniforms(u_resample, B, bad, stream);
      return e;
    });
    if (st != CLM_OK) return st;
  }
  clm::VerifyArgs a{target_logits, draft_probs, draft_tokens, u_accept, u_resample, temperature,
                    B, K, V, out_tokens, num_emitted, bonus};
  return hip_status(clm::launch_spec_verify(a, stream));
}

int clm_spec_verify(const float* target_logits, const float* draft_probs,
                    const int32_t* draft_tokens, const float* u_accept, const float* u_resample,
                    float temperature, int B, int K, int V, int32_t* out_tokens,
                    int32_t* num_emitted, hipStream_t stream) {
  return spec_verify_impl(target_logits, draft_probs, draft_tokens, u_accept, u_resample, temperature,
                          B, K, V, out_tokens, num_emitted, 0, stream);
}

int clm_spec_verify_bonus(const float* target_logits, const float* draft_probs,
                          const int32_t* draft_tokens, const float* u_accept, const float* u_resample,
                          float temperature, int B, int K, int V, int32_t* out_tokens,
                          int32_t* num_emitted, hipStream_t stream) {
  return spec_verify_impl(target_logits, draft_probs, draft_tokens, u_accept, u_resample, temperature,
                          B, K, V, out_tokens, num_emitted, 1, stream);
}

}  // extern "C"
