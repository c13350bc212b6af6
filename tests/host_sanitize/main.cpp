// Host-side validation of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point called with good and bad
// host arguments (sizes at and past their limits, null and misaligned
// pointers, overflowing products), checking the status each returns.  No
// GPU is involved: pointers are never dereferenced by the host code, and a
// call that passes validation reaches a stub that reports no device.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "../../include/clm.h"

static int failures = 0;
#define EXPECT(call, want)                                                                       \
  do {                                                                                           \
    const int got_ = (call);                                                                     \
    if (got_ != (want)) {                                                                        \
      std::printf("line %d: %s returned %d (%s), expected %d\n", __LINE__, #call, got_,          \
                  clm_status_string(got_), (int)(want));                                         \
      ++failures;                                                                                \
    }                                                                                            \
  } while (0)

int main() {
  void* P = reinterpret_cast<void*>(uintptr_t(0x100000));   // aligned, never dereferenced
  void* Pm = reinterpret_cast<void*>(uintptr_t(0x100008));  // 8-byte aligned only
  int32_t* I = static_cast<int32_t*>(P);
  float* F = static_cast<float*>(P);
  const hipStream_t S = nullptr;
  const int INV = CLM_ERR_INVALID_ARG, UNS = CLM_ERR_UNSUPPORTED, CAP = CLM_ERR_CAPACITY,
            WS = CLM_ERR_WORKSPACE, HIP = CLM_ERR_HIP;

  // status strings, version, checked-mode switch
  for (int s = 1; s >= -7; --s) EXPECT((int)(std::strlen(clm_status_string(s)) > 0), 1);
  EXPECT(clm_version() >= 200, 1);
  const int prev = clm_set_checked(1);
  EXPECT(clm_set_checked(0), 1);
  clm_set_checked(prev);

  // append
  EXPECT(clm_kv_cache_append(nullptr, P, P, P, I, 8, I, 2, 1, 8, 128, 16, 100, CLM_BF16, S), INV);
  EXPECT(clm_kv_cache_append(P, P, P, P, I, 8, I, 0, 1, 8, 128, 16, 100, CLM_BF16, S), INV);
  EXPECT(clm_kv_cache_append(Pm, P, P, P, I, 8, I, 2, 1, 8, 128, 16, 100, CLM_BF16, S), INV);
  EXPECT(clm_kv_cache_append(P, P, P, P, I, 8, I, 2, 1, 8, 96, 16, 100, CLM_BF16, S), UNS);
  EXPECT(clm_kv_cache_append(P, P, P, P, I, 8, I, 2, 129, 8, 128, 16, 100, CLM_BF16, S), CAP);
  EXPECT(clm_kv_cache_append(P, P, P, P, I, 8, I, 2, 1, 8, 128, 16, 100, (clm_dtype)7, S), UNS);
  EXPECT(clm_kv_cache_append(P, P, P, P, I, 8, I, 2, 1, 8, 128, 16, 100, CLM_BF16, S), HIP);
  EXPECT(clm_kv_cache_append(P, P, P, P, I, std::numeric_limits<int>::max(), I, std::numeric_limits<int>::max(),
                             1, std::numeric_limits<int>::max(), 128, 256, 100, CLM_BF16, S), UNS);
  EXPECT(clm_rope_kv_cache_append(P, P, P, P, P, I, 8, I, I, std::nanf(""), 4, 1, 16, 8, 128, 16, 64,
                                  CLM_BF16, S), INV);
  EXPECT(clm_rope_kv_cache_append(P, P, P, P, P, I, 8, I, I, 1e6f, 4, 1, 12, 8, 128, 16, 64, CLM_BF16, S), INV);
  EXPECT(clm_rope_kv_cache_append(P, P, P, P, P, I, 8, I, I, 1e6f, 4, 1, 16, 8, 128, 16, 64, CLM_BF16, S), HIP);
  EXPECT(clm_kv_cache_append_fp8(P, P, P, P, F, F, I, 8, I, 2, 1, 8, 64, 16, 100, S), HIP);
  EXPECT(clm_kv_cache_append_fp8(P, P, P, P, nullptr, F, I, 8, I, 2, 1, 8, 64, 16, 100, S), INV);
  EXPECT(clm_rope_kv_cache_append_fp8(P, P, P, P, P, F, F, I, 8, I, I, 1e6f, 2, 1, 16, 8, 64, 16, 100, S), HIP);
  EXPECT(clm_rope_kv_cache_append_fp8(nullptr, P, P, P, P, F, F, I, 8, I, I, 1e6f, 2, 1, 16, 8, 64, 16, 100, S), INV);
  EXPECT(clm_rope_kv_cache_append_fp8(P, P, P, P, P, F, F, I, 8, I, I, 1e6f, 2, 1, 12, 8, 64, 16, 100, S), INV);
  EXPECT(clm_rope_kv_cache_append_fp8(P, P, P, P, P, F, F, I, 8, I, I, 1e6f, 2, 1, 16, 8, 96, 16, 100, S), UNS);

  // attention: the workspace query, then the call
  const size_t need = clm_decode_attention_workspace_size(4, 1, 16, 8, 128, 1000);
  EXPECT((int)(need > 0), 1);
  EXPECT((int)clm_decode_attention_workspace_size(4096, 1, 32, 32, 128, 100), 0);
  EXPECT((int)clm_decode_attention_workspace_size(4, 1, 16, 8, 128, std::numeric_limits<int>::max()) > 0, 1);
  EXPECT(clm_decode_attention(P, P, P, I, 64, I, 1000, P, 4, 1, 16, 8, 128, 16, 300, 0.088f, CLM_BF16, P,
                              need - 1, S), WS);
  EXPECT(clm_decode_attention(P, P, P, I, 64, I, 1000, P, 4, 1, 16, 8, 128, 16, 300, INFINITY, CLM_BF16, P,
                              need, S), INV);
  EXPECT(clm_decode_attention(P, P, P, I, 64, I, 1000, P, 4, 6, 32, 8, 128, 16, 300, 0.088f, CLM_BF16, P,
                              need, S), UNS);
  EXPECT(clm_decode_attention(P, P, P, I, 64, I, 1000, P, 4, 1, 16, 8, 128, 16, 300, 0.088f, CLM_BF16, P,
                              need, S), HIP);
  EXPECT(clm_decode_attention_noalloc(P, P, P, I, 4096, I, 65536, P, 256, 1, 16, 8, 128, 16, 1 << 20, 0.088f,
                                      CLM_BF16, S), WS);
  EXPECT(clm_decode_attention_noalloc(P, P, P, I, 64, I, 1000, P, 4, 1, 16, 8, 128, 16, 300, 0.088f, CLM_BF16,
                                      S), HIP);
  EXPECT(clm_decode_attention_fp8(P, P, P, F, F, I, 64, I, 1000, P, 4, 1, 16, 8, 128, 16, 300, 0.088f, P, need,
                                  S), HIP);
  EXPECT(clm_decode_attention_fp8(P, P, P, static_cast<float*>(Pm), F, I, 64, I, 1000, P, 4, 1, 16, 8, 128, 16,
                                  300, 0.088f, P, need, S), INV);

  // head
  const void* Ws[3] = {P, P, P};
  EXPECT((int)clm_codebook_head_workspace_size(256, 2048, 16384, 1, CLM_BF16), 0);
  EXPECT(clm_codebook_head(P, Ws, 3, nullptr, F, 64, 2048, 4096, CLM_BF16, nullptr, 0, S), INV);
  EXPECT(clm_codebook_head(P, Ws, 1, nullptr, F, 70000, 2048, 4096, CLM_BF16, nullptr, 0, S), UNS);
  EXPECT(clm_codebook_head(P, Ws, 1, nullptr, F, 64, 2048, 4096, CLM_BF16, Pm, 64, S), WS);
  EXPECT(clm_codebook_head(P, Ws, 3, I, F, 64, 2048, 4096, CLM_BF16, nullptr, 0, S), HIP);
  EXPECT(clm_codebook_head(P, Ws, 1, nullptr, F, 1, 256, 4096, CLM_F32, nullptr, 0, S), HIP);
  EXPECT(clm_codebook_head_mlp(P, Ws, Ws, 1, nullptr, P, F, 16, 2048, 4096, 4096, CLM_BF16, nullptr, 0, S), HIP);
  EXPECT(clm_codebook_head_mlp(P, Ws, Ws, 1, nullptr, P, F, 16, 2048, 4000, 4096, CLM_BF16, nullptr, 0, S), UNS);

  // token choice and verification
  EXPECT(clm_sample_or_argmax(F, 4, 100, 99, nullptr, nullptr, nullptr, I, S), INV);
  EXPECT(clm_sample_or_argmax(F, 4, (1 << 20) + 1, (1 << 20) + 1, nullptr, nullptr, nullptr, I, S), UNS);
  EXPECT(clm_sample_or_argmax(F, 4, 100, 128, F, F, I, I, S), HIP);
  EXPECT(clm_spec_verify(F, F, I, F, F, -0.1f, 4, 6, 4096, I, I, S), INV);
  EXPECT(clm_spec_verify(F, F, I, F, F, 0.7f, 4, 17, 4096, I, I, S), UNS);
  EXPECT(clm_spec_verify_bonus(F, F, I, F, F, 0.7f, 4, 16, 4096, I, I, S), UNS);
  EXPECT(clm_spec_verify(F, F, I, F, F, 0.7f, 4, 6, 4096, I, I, S), HIP);

  // decode loop
  int32_t sizes[3] = {16, 64, 256};
  EXPECT(clm_pick_bucket(sizes, 3, 17), 1);
  EXPECT(clm_pick_bucket(sizes, 3, 300), -1);
  EXPECT(clm_advance_lengths(nullptr, I, nullptr, nullptr, 4, 1, S), INV);
  EXPECT(clm_advance_lengths(I, I, nullptr, nullptr, 4, 1, S), HIP);
  clm_decode_step_desc d;
  std::memset(&d, 0, sizeof d);
  d.B = 4; d.Kq = 1; d.H_q = 16; d.H_kv = 8; d.D = 128; d.block_size = 16; d.num_blocks = 64; d.max_blocks = 8;
  d.max_kv_len = 128; d.G = 1; d.V = 4096; d.dt = CLM_BF16;
  d.k_cache = d.v_cache = P; d.block_table = I; d.len_before = d.kv_len = I; d.k_new = d.v_new = P; d.q = P;
  d.W = Ws; d.o = P; d.logits = F; d.tokens = I; d.mode = 0;
  clm_decode_loop* loop = nullptr;
  EXPECT(clm_decode_loop_create(&d, 0, &loop), INV);
  EXPECT(clm_decode_loop_create(nullptr, 4, &loop), INV);
  d.mode = 2;
  EXPECT(clm_decode_loop_create(&d, 4, &loop), INV);
  d.mode = 3;                                              // bonus verification needs Kq >= 2
  d.draft_probs = F; d.draft_tokens = I; d.u_accept = F; d.u_resample = F; d.out_tokens = I; d.num_emitted = I;
  EXPECT(clm_decode_loop_create(&d, 4, &loop), INV);
  d.draft_probs = nullptr; d.draft_tokens = nullptr; d.u_accept = nullptr; d.u_resample = nullptr;
  d.out_tokens = nullptr; d.num_emitted = nullptr;
  d.mode = 0;
  d.k_scale = F;                                           // FP8 cache: one scale array alone
  EXPECT(clm_decode_loop_create(&d, 4, &loop), INV);
  d.v_scale = F;                                           // no caller workspace
  EXPECT(clm_decode_loop_create(&d, 4, &loop), UNS);
  d.attn_workspace = P; d.attn_workspace_bytes = 1 << 20;
  EXPECT(clm_decode_loop_create(&d, 4, &loop), HIP);       // FP8 loop: no device either
  d.k_scale = d.v_scale = nullptr; d.attn_workspace = nullptr; d.attn_workspace_bytes = 0;
  d.W2 = Ws; d.F = 4096;                                   // two-layer head without its activation scratch
  EXPECT(clm_decode_loop_create(&d, 4, &loop), INV);
  d.act = P; d.dt = CLM_F32;                               // two-layer head takes bf16 only
  EXPECT(clm_decode_loop_create(&d, 4, &loop), UNS);
  d.W2 = nullptr; d.F = 0; d.act = nullptr; d.dt = CLM_BF16;
  EXPECT(clm_decode_loop_create(&d, 4, &loop), HIP);       // no device: capture cannot start
  EXPECT((int)(loop == nullptr), 1);
  EXPECT(clm_decode_loop_launch(nullptr, S), INV);
  EXPECT(clm_decode_loop_destroy(nullptr), INV);

  std::printf("%s: %d mismatches\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
