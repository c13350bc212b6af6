// Internal host-side interface between the C ABI (abi.cpp) and the kernel
// translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace clm {

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const int32_t* len_before;
  int max_blocks, B, T_new, H_kv, D, block_size, num_blocks;
  bool bf16;
};
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s);

struct RopeAppendArgs {
  void* q;                     // [B, T_new, H_q, D], rotated in place
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* len_before;
  const int32_t* positions;    // [B, T_new] logical positions
  float rope_base;
  int B, T_new, H_q, H_kv, D, block_size, num_blocks;
  bool bf16;
};
hipError_t launch_rope_kv_append(const RopeAppendArgs& a, hipStream_t s);

struct Fp8AppendArgs {
  const void* k_new;           // [B, T_new, H_kv, D] bf16
  const void* v_new;
  void* k_cache;               // [num_blocks, H_kv, D/8, bs, 8] E4M3 bytes
  void* v_cache;               // [num_blocks, H_kv, D, bs] E4M3 bytes
  float* k_scale;              // [num_blocks, H_kv, bs]
  float* v_scale;
  const int32_t* block_table;
  const int32_t* len_before;
  int max_blocks, B, T_new, H_kv, D, block_size, num_blocks;
  // rotary embedding at logical positions (q == nullptr: none)
  void* q = nullptr;                  // [B, T_new, H_q, D] bf16, rotated in place
  const int32_t* positions = nullptr; // [B, T_new]
  float rope_base = 0.f;
  int H_q = 0;
};
hipError_t launch_fp8_kv_append(const Fp8AppendArgs& a, hipStream_t s);

struct AttnPlan {
  int split;        // tokens per work item (multiple of 64)
  int max_splits;   // ceil(max_kv_len / split)
  int nr;           // query rows per KV head = G * Kq
  int nr_tmpl;      // compiled row capacity (>= nr)
  size_t ml_offset, acc_offset, total_bytes;
};
// Deterministic function of the sizes; the workspace query and the call use it.
bool plan_decode_attention(int B, int Kq, int H_q, int H_kv, int D, int max_kv_len, AttnPlan* p);

struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* kv_len;
  void* o;
  void* workspace;
  int max_blocks, max_kv_len, B, Kq, H_q, H_kv, D, block_size, num_blocks;
  float scale;
  bool bf16;
  const float* k_scale = nullptr;   // non-null: E4M3 K/V cache with per-row scales
  const float* v_scale = nullptr;
};
hipError_t launch_decode_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t s);

// The library's static scratch for attention split partials (one copy per
// GPU): its size, and its device address on the current device (looked up
// once per device with hipGetSymbolAddress).
constexpr size_t kAttentionScratchBytes = (size_t)32 << 20;
hipError_t attention_scratch(void** ptr);

struct HeadArgs {
  const void* h;
  const void* W[8];
  int G;
  const int32_t* head_id;
  float* logits;
  int M, d, V;
  bool bf16;
  uint16_t* act;   // non-null: write bf16(Mish(h W^T)) here ([M, V]) instead of logits
};
// Tile plan of the bf16 head (a deterministic function of M, V, G).
struct HeadPlan {
  int nv, mr, nw;            // codebook entries and rows per workgroup, waves
  int row_chunks, nvt, nvt_pad;
  size_t workspace_bytes;    // scratch the plan needs (none for these tiles)
};
HeadPlan plan_codebook_head(int M, int V, int G);
hipError_t launch_codebook_head(const HeadArgs& a, hipStream_t s);

struct SampleArgs {
  const float* logits;
  int M, V, ld;
  const float* temperature;
  const float* uniforms;
  const int32_t* vocab_valid;
  int32_t* tokens;
};
hipError_t launch_sample_or_argmax(const SampleArgs& a, hipStream_t s);

struct VerifyArgs {
  const float* target_logits;
  const float* draft_probs;
  const int32_t* draft_tokens;
  const float* u_accept;
  const float* u_resample;
  float temperature;
  int B, K, V;
  int32_t* out_tokens;
  int32_t* num_emitted;
  int bonus;   // 1: K+1 target rows and out rows, a bonus draw after K accepts
};
hipError_t launch_spec_verify(const VerifyArgs& a, hipStream_t s);

// Checked mode on (CLM_CHECK / clm_set_checked), for calls that must refuse it.
bool checked_mode();

// Decode loop: lengths (and positions) += num_emitted[b] (or T_new) per stream.
hipError_t launch_advance(int32_t* len_before, int32_t* kv_len, int32_t* positions, const int32_t* num_emitted,
                          int B, int T_new, hipStream_t s);

// Checked mode: validators add the number of bad entries to *bad (device int,
// zeroed by the caller); check_counter gives the library's static counter on
// the current device.
hipError_t check_counter(int** ptr);
hipError_t launch_check_lengths(const int32_t* len, int n, int lo, int hi, int* bad, hipStream_t s);
hipError_t launch_check_block_table(const int32_t* bt, const int32_t* len, int B, int max_blocks,
                                    int len_add, int block_size, int num_blocks, int* bad,
                                    hipStream_t s);
hipError_t launch_check_ints(const int32_t* x, int n, int lo, int hi, int* bad, hipStream_t s);
hipError_t launch_check_uniforms(const float* u, int n, int* bad, hipStream_t s);

}  // namespace clm
