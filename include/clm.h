/*
 * clm.h - C ABI of libclm.so: one batched autoregressive decode step of a
 * codec-language-model text-to-speech generator, as hand-written HIP kernels
 * for AMD Instinct MI355X (gfx950).
 *
 * The step (TTS Serving, in depth, "Token generation under a frame budget":
 * after a prefill, the generator runs one decode step per audio frame and each
 * step reads the KV cache; continuous batching over a paged cache):
 *
 *   clm_kv_cache_append    write the step's new K/V rows into the paged cache
 *   clm_rope_kv_cache_append  the same with rotary position embedding at
 *                          logical positions applied to the new keys and queries
 *   clm_decode_attention   single- or K-query GQA attention over each stream's
 *                          ragged cache (split-KV flash decoding)
 *   clm_kv_cache_append_fp8, clm_decode_attention_fp8
 *                          the same two calls for an FP8 (E4M3) cache
 *   clm_rope_kv_cache_append_fp8  the rotary append into the FP8 cache
 *   clm_codebook_head      codebook logit projection, optionally grouped by
 *                          stage (one weight matrix per stage)
 *   clm_codebook_head_mlp  the two-layer (d -> F -> Mish -> V) form of that head
 *   clm_sample_or_argmax   greedy argmax or temperature sampling per row
 *   clm_spec_verify        speculative accept/reject of K drafted tokens
 *   clm_spec_verify_bonus  the same with a bonus token after K accepts
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers.  Every array argument is DEVICE memory owned by the caller, except
 *   where a comment says "host".  The library keeps no per-call state, never
 *   allocates in these calls and never frees caller memory.
 * Asynchrony.  A call validates its host-visible arguments, enqueues its
 *   kernels on `stream` (NULL = the null stream) and returns.  It never
 *   synchronises and never reads device memory on the host, so a fixed-shape
 *   step can be captured in a HIP graph.  The one exception is checked mode
 *   (on when the environment variable CLM_CHECK is set to a value other than
 *   "0" at load, and switched with clm_set_checked): each call then first
 *   runs a validator over its device-resident indices (lengths, block ids,
 *   head ids, tokens, uniforms), synchronises, and returns
 *   CLM_ERR_DEVICE_DATA without launching anything if one is out of range.
 *   Checked mode counts bad entries in a 4-byte counter in the library's
 *   static device memory (no allocation), cleared with hipMemsetAsync before
 *   each validation; it synchronises, so it is for tests and debugging, not
 *   for graph capture.
 * Errors.  A call returns CLM_OK or a negative clm_status.  Host-visible
 *   arguments are checked before any HIP call: a call that returns an error
 *   other than CLM_ERR_HIP has enqueued nothing.  Device-resident values are
 *   trusted outside checked mode; kernels still clamp every block-table entry,
 *   length and head id they read into range, so bad device data gives wrong
 *   numbers, not out-of-bounds memory accesses.
 * Element types.  q, K, V, o, h and W share one element type per call
 *   (clm_dtype).  Logits, probabilities, temperatures and uniforms are always
 *   float32; tokens, lengths and indices are int32.
 * Layouts are row-major (C order) with the shapes given; "[a, b]" means b is
 *   contiguous.
 */
#ifndef CLM_H
#define CLM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { CLM_F32 = 0, CLM_BF16 = 1 } clm_dtype;

typedef enum {
  CLM_OK = 0,
  CLM_ERR_INVALID_ARG = -1,  /* null pointer, non-positive or inconsistent size   */
  CLM_ERR_UNSUPPORTED = -2,  /* valid but not implemented (D, dtype, group size)  */
  CLM_ERR_CAPACITY = -3,     /* append would overflow a stream's block-table row  */
  CLM_ERR_WORKSPACE = -4,    /* workspace missing or smaller than required        */
  CLM_ERR_HIP = -5,          /* a HIP runtime call failed (launch, query)         */
  CLM_ERR_DEVICE_DATA = -6   /* checked mode found an out-of-range device value   */
} clm_status;

/* Human-readable name of a clm_status value (static string). */
const char* clm_status_string(int status);

/* ABI version: major*10000 + minor*100 + patch. */
int clm_version(void);

/*
 * Checked mode on (on != 0) or off for every later call of this process, on
 * every GPU; returns the previous setting (0 or 1).  The initial setting
 * comes from CLM_CHECK.  Host-only: no HIP call.  Calls already running on
 * other host threads keep the setting they started with.
 */
int clm_set_checked(int on);

/* --------------------------------------------------------------------------
 * KV cache layout (paged).  Optimizing Streaming Text-to-Speech Models for
 * Sub-50 Millisecond Latency, "Dynamic Token-Level Batching": the cache is a
 * static pool of fixed-size blocks (16 tokens there) that streams take from a
 * global free list and give back when done; the free list is the caller's.
 *
 *   k_cache [num_blocks, H_kv, block_size, D]   one key row per token slot
 *   v_cache [num_blocks, H_kv, D, block_size]   values TRANSPOSED inside a block
 *   block_table [B, max_blocks] int32            stream b's logical block p
 *                                                (token positions
 *                                                [p*block_size, (p+1)*block_size))
 *                                                lives in pool block
 *                                                block_table[b*max_blocks + p]
 * Values are stored transposed so that the attention kernels read, for one
 * head dimension, consecutive tokens as one contiguous run (the operand
 * layout the matrix cores and the dot-product loop want for P.V).
 * block_size must be a multiple of 16 in [16, 256].
 * ------------------------------------------------------------------------ */

/*
 * Append T_new new rows per stream at positions len_before[b] .. len_before[b]+T_new-1.
 *   k_new, v_new  [B, T_new, H_kv, D]      rows to write (element type dt)
 *   k_cache, v_cache                       pool, layout above; updated in place
 *   block_table   [B, max_blocks]          must map every written position
 *   len_before    [B] int32                tokens already in each stream
 * Every other cache slot is left untouched; the result is bit-exact copies.
 * Errors: INVALID_ARG (null, B/T_new/H_kv/D/max_blocks/num_blocks < 1),
 *   UNSUPPORTED (D not 64 or 128, block_size not a multiple of 16 in
 *   [16,256], unknown dt), CAPACITY (T_new > max_blocks*block_size).
 * Rows whose position falls outside the block table, or whose block id is
 * outside [0, num_blocks), are skipped (checked mode reports them).
 */
int clm_kv_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int32_t* block_table, int max_blocks, const int32_t* len_before,
                        int B, int T_new, int H_kv, int D, int block_size, int num_blocks,
                        clm_dtype dt, hipStream_t stream);

/*
 * The append with rotary position embedding at logical positions fused in
 * (TontaubeV1: positions are logical coordinates and rotary attention depends
 * only on their differences - the vLLM adapters add one constant to every
 * prefill coordinate; the speculative-decoding blog, "Engine-Level
 * Optimizations with TensorRT-LLM": rotary embedding fused with the KV-cache
 * write).  For new token t of stream b at logical position p = positions[b,t]:
 *     theta_i = rope_base^(-2i/D),  a_i = p * theta_i      (fp64)
 *     (x_i, x_{i+D/2}) -> (x_i cos a_i - x_{i+D/2} sin a_i,
 *                          x_i sin a_i + x_{i+D/2} cos a_i)   i < D/2
 * is applied to the key row as it is written into its cache slot (the slot
 * is len_before[b] + t, as in clm_kv_cache_append), and to q[b,t,:,:] in
 * place; values are copied unrotated.
 *   q          [B, T_new, H_q, D]   queries of the step's new tokens, rotated in place
 *   positions  [B, T_new] int32     logical positions (any integers)
 *   rope_base  host float > 1       (e.g. 1e6)
 *   other arguments as clm_kv_cache_append; k_new is not modified
 * Arithmetic: angles, cos and sin in fp64; rotation in fp32; results rounded
 * to dt once.
 * Errors: as clm_kv_cache_append, plus INVALID_ARG for null q or positions,
 *   H_q % H_kv != 0, or rope_base not finite or <= 1.
 */
int clm_rope_kv_cache_append(void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* block_table, int max_blocks, const int32_t* len_before,
                             const int32_t* positions, float rope_base, int B, int T_new, int H_q,
                             int H_kv, int D, int block_size, int num_blocks, clm_dtype dt,
                             hipStream_t stream);

/*
 * Bytes of workspace clm_decode_attention needs for these sizes (0 on a size
 * error).  max_kv_len bounds kv_len[b] for every stream of the call.
 */
size_t clm_decode_attention_workspace_size(int B, int Kq, int H_q, int H_kv, int D,
                                           int max_kv_len);

/*
 * Decode attention, one step, all streams.  For stream b, query j in [0,Kq)
 * and query head h (H_q heads, H_kv KV heads, group G = H_q/H_kv):
 *     n   = kv_len[b] - (Kq-1-j)          keys visible to query j (a causal
 *                                         block of Kq queries: the last query
 *                                         sees every key, including the rows
 *                                         appended this step)
 *     kvh = h / G                         consecutive query heads share a KV head
 *     o[b,j,h,:] = softmax(scale * q[b,j,h,:] . K[0:n,kvh,:]) . V[0:n,kvh,:]
 * (Speculative Decoding for Acoustic Tokens: one target pass scores the K
 * drafted positions, i.e. Kq = K queries with causal visibility.)
 *   q          [B, Kq, H_q, D]        queries (already position-rotated)
 *   k_cache, v_cache, block_table     paged cache, layout above
 *   kv_len     [B] int32              visible keys of the last query, >= Kq,
 *                                     <= max_kv_len
 *   max_kv_len                        host bound on kv_len (sizes the split plan)
 *   o          [B, Kq, H_q, D]        output, element type dt
 *   scale                             score scale (1/sqrt(D) for standard attention)
 *   workspace  >= clm_decode_attention_workspace_size(...) bytes, 256-byte
 *              aligned, caller-owned scratch for per-split partial results;
 *              no initial contents are needed.  Calls that share a workspace
 *              must be ordered on one stream.
 * Arithmetic: fp32 dot products, exponentials, online softmax and
 * accumulation; o rounded to dt once.  Splits are fixed token ranges of each
 * stream; streams longer than one split are merged by a second kernel in
 * split order, so results are the same from run to run and do not depend on
 * the order in which workgroups finish, nor on the other streams of the
 * batch.
 * Errors: INVALID_ARG (null, sizes < 1, H_q % H_kv != 0, max_kv_len < Kq,
 *   scale not finite), UNSUPPORTED (D not 64/128, G*Kq > 16, B > 4096,
 *   B*H_kv > 65536, block_size as for append, unknown dt), WORKSPACE (too
 *   small or misaligned).
 */
int clm_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, int max_blocks, const int32_t* kv_len,
                         int max_kv_len, void* o, int B, int Kq, int H_q, int H_kv, int D,
                         int block_size, int num_blocks, float scale, clm_dtype dt,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * clm_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops that must not call hipMalloc,
 * harnesses that forbid it).  The same computation, kernels and results as
 * clm_decode_attention with the same arguments, but with no workspace: the
 * split partials go to the library's own static device scratch of
 * 32 MiB (33554432 bytes) per GPU, held from the first use on that GPU
 * until the process ends.  The call allocates nothing: the scratch's device
 * address is looked up once per device (hipGetSymbolAddress) and reused.
 * Every call on one GPU shares that GPU's scratch, so calls that overlap in
 * time on one GPU (other streams, other host threads) race and give wrong
 * results; order them on one stream.  The scratch needs no initial contents.
 * Errors: those of clm_decode_attention, with WORKSPACE when
 * clm_decode_attention_workspace_size(B, Kq, H_q, H_kv, D, max_kv_len) is
 * above 32 MiB (the check precedes any HIP call).
 */
int clm_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, int max_blocks, const int32_t* kv_len,
                                 int max_kv_len, void* o, int B, int Kq, int H_q, int H_kv, int D,
                                 int block_size, int num_blocks, float scale, clm_dtype dt,
                                 hipStream_t stream);

/*
 * FP8 (E4M3) KV cache (the speculative-decoding blog, "Engine-Level
 * Optimizations with TensorRT-LLM": FP8 quantization of the target model's
 * attention; here applied to the KV cache every step reads, halving its
 * bytes).  One byte per element, plus one fp32 scale per (block, KV head,
 * slot) for keys and for values:
 *   k_cache [num_blocks, H_kv, D/8, block_size, 8]  E4M3 codes (uint8): keys
 *           in 8-dimension groups, each group of a block's keys contiguous
 *   v_cache [num_blocks, H_kv, D, block_size]  E4M3 codes, transposed per block
 *   k_scale, v_scale [num_blocks, H_kv, block_size] float32, 16-byte aligned
 * E4M3: 4 exponent bits (bias 7), 3 mantissa bits, largest 448, no
 * infinities.  A stored row x (D values of one token and KV head) is
 *   scale = max|x| / 448 (1 if all zero),  code_i = E4M3(clamp(x_i / scale, +-448))
 * rounded to nearest with ties to the even code, and reads back as
 * decode(code_i) * scale.
 *
 * clm_kv_cache_append_fp8: clm_kv_cache_append for this cache; k_new, v_new
 * are bf16 [B, T_new, H_kv, D], quantized as written.  Errors as
 * clm_kv_cache_append (dt is bf16 implicitly).
 */
int clm_kv_cache_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            float* k_scale, float* v_scale, const int32_t* block_table, int max_blocks,
                            const int32_t* len_before, int B, int T_new, int H_kv, int D, int block_size,
                            int num_blocks, hipStream_t stream);

/*
 * clm_rope_kv_cache_append for the FP8 cache: the rotary embedding of
 * clm_rope_kv_cache_append (same angles, fp64, and the same fp32 rotation) is
 * applied to each new key row, which is then quantized from its fp32 values
 * as clm_kv_cache_append_fp8 quantizes a row; values are quantized
 * unrotated; q (bf16) is rotated in place exactly as clm_rope_kv_cache_append
 * rotates it.  q, k_new, v_new bf16; caches and scales as
 * clm_kv_cache_append_fp8.  Errors as clm_kv_cache_append_fp8, plus those
 * clm_rope_kv_cache_append adds (null q or positions, H_q % H_kv != 0,
 * rope_base not finite or <= 1, q not 16-byte aligned).
 */
int clm_rope_kv_cache_append_fp8(void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 float* k_scale, float* v_scale, const int32_t* block_table, int max_blocks,
                                 const int32_t* len_before, const int32_t* positions, float rope_base, int B,
                                 int T_new, int H_q, int H_kv, int D, int block_size, int num_blocks,
                                 hipStream_t stream);

/*
 * clm_decode_attention over the FP8 cache: q and o bf16, the same visibility,
 * scale and split plan (workspace: clm_decode_attention_workspace_size).
 * Keys and values are decoded to bf16 exactly in registers; scores are
 * multiplied by the key scales and probabilities by the value scales, all in
 * fp32.  Errors as clm_decode_attention, plus INVALID_ARG for a null or
 * misaligned scale array.
 */
int clm_decode_attention_fp8(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                             const float* v_scale, const int32_t* block_table, int max_blocks,
                             const int32_t* kv_len, int max_kv_len, void* o, int B, int Kq, int H_q, int H_kv,
                             int D, int block_size, int num_blocks, float scale, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Codebook logit projection (TontaubeV1, audio head paragraph: each stage owns
 * a head that maps the transformer state onto that stage's codebook; codec
 * paragraph: 16,384 semantic / 4,096 acoustic entries).  No bias.
 *     logits[r, v] = sum_k h[r, k] * W_{g(r)}[v, k],   g(r) = head_id[r] (or 0)
 *   h        [M, d]                   head input (element type dt)
 *   W        host array of G device pointers, each [V, d] (element type dt)
 *   head_id  [M] int32 in [0, G), or NULL when G == 1
 *   logits   [M, V] float32           output
 *   workspace, workspace_bytes        caller-owned scratch of at least
 *            clm_codebook_head_workspace_size(M, d, V, G, dt) bytes, 256-byte
 *            aligned when non-NULL.  NULL with 0 bytes is valid when that size
 *            is 0, which it is for every tile plan of this version; the
 *            argument is part of the call so that a plan needing scratch
 *            (partial sums of a split k range) changes no signature.
 * Each W_g is streamed from memory once per call for up to 128 rows of its
 * group; more rows are taken in chunks whose workgroups read the same W tile
 * close together in time, so it comes from memory about once.
 * Arithmetic (bf16): products of bf16 values accumulated in fp32 in two
 * chains, over the even and over the odd 32-wide k blocks, added once at the
 * end; a row's logits do not depend on the other rows of the call (nor on M,
 * G or the tile plan).  fp32: one fp32 dot product per logit.
 * Errors: INVALID_ARG (null, sizes < 1, G > 8, head_id NULL with G > 1,
 *   h or a W not 16-byte aligned), UNSUPPORTED (bf16 with d % 128 != 0, f32
 *   with d % 4 != 0, M > 65536, unknown dt), WORKSPACE (smaller than the
 *   query's size, or non-NULL and misaligned).
 */
size_t clm_codebook_head_workspace_size(int M, int d, int V, int G, clm_dtype dt);
int clm_codebook_head(const void* h, const void* const* W, int G, const int32_t* head_id,
                      float* logits, int M, int d, int V, clm_dtype dt, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * Two-layer audio head (TontaubeV1, audio head paragraph: each stage's head
 * widens the transformer state to 4,096, applies a Mish nonlinearity and
 * projects to that stage's audio vocabulary).  No biases.
 *     act[r, f]    = bf16( Mish( sum_k h[r, k] * W1_{g(r)}[f, k] ) )
 *     logits[r, v] = sum_f act[r, f] * W2_{g(r)}[v, f]
 *     Mish(x) = x * tanh(softplus(x)),  g(r) = head_id[r] (or 0)
 *   h        [M, d] bf16
 *   W1, W2   host arrays of G device pointers: W1_g [F, d], W2_g [V, F], bf16
 *   head_id  [M] int32 in [0, G), or NULL when G == 1
 *   act      [M, F] bf16, caller-owned: written with the widened activation
 *            (rounded to nearest even), then read by the second product
 *   logits   [M, V] float32 output
 *   workspace, workspace_bytes   as for clm_codebook_head, sized by
 *            clm_codebook_head_mlp_workspace_size(M, d, F, V, G)
 * Two kernel launches on `stream`: the first product with Mish fused into its
 * epilogue, then the second.  Arithmetic: each product as in
 * clm_codebook_head (bf16 products, fp32 accumulation in two chains); Mish in
 * fp32.
 * Errors: INVALID_ARG (null, sizes < 1, G > 8, head_id NULL with G > 1, h, act
 *   or a weight not 16-byte aligned), UNSUPPORTED (dt not bf16, d or F not a
 *   multiple of 128, M > 65536), WORKSPACE (as for clm_codebook_head).
 */
size_t clm_codebook_head_mlp_workspace_size(int M, int d, int F, int V, int G);
int clm_codebook_head_mlp(const void* h, const void* const* W1, const void* const* W2, int G,
                          const int32_t* head_id, void* act, float* logits, int M, int d, int F, int V,
                          clm_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One token per row (TontaubeV1 decodes later stages greedily; Section 3.3
 * masks logits outside the stage's target vocabulary at sampling time).
 *   logits       [M, ld] float32, first V columns used (ld >= V)
 *   temperature  [M] float32 >= 0, or NULL (every row greedy)
 *   uniforms     [M] float32 in [0, 1); required when temperature != NULL
 *   vocab_valid  [M] int32 in [1, V], or NULL: columns >= vocab_valid[r] are excluded
 *   tokens       [M] int32 output
 * T = 0: the lowest index of the largest logit.
 * T > 0: z = logit / T (fp32 division), e_i = exp(z_i - max z),
 *        token = min{ i : u*S < e_0 + ... + e_i } with S = sum e  (inverse CDF
 *        in ascending index order); if rounding leaves no such i, the last
 *        index with e_i > 0.
 * Errors: INVALID_ARG (null logits/tokens, M/V < 1, ld < V, uniforms NULL with
 *   temperature set), UNSUPPORTED (V > 1<<20).
 */
int clm_sample_or_argmax(const float* logits, int M, int V, int ld, const float* temperature,
                         const float* uniforms, const int32_t* vocab_valid, int32_t* tokens,
                         hipStream_t stream);

/*
 * Speculative verification (Speculative Decoding for Acoustic Tokens).  For
 * each stream independently, i = 0..K-1:
 *     p = softmax(target_logits[b,i,:] / T)   (T = 0: one-hot at the argmax)
 *     x = draft_tokens[b,i],  q = draft_probs[b,i,x]
 *     accept iff q > 0 and u_accept[b,i] < p[x] / q   -> emit x, continue
 *     else emit the inverse-CDF draw (ascending index order) at u_resample[b]
 *          from max(p - draft_probs[b,i,:], 0) (from p if that is all zero)
 *          and stop.
 * No bonus token follows K accepts.
 *   target_logits [B, K, V] float32,  draft_probs [B, K, V] float32
 *   draft_tokens  [B, K] int32 in [0, V)
 *   u_accept      [B, K] float32 in [0,1),  u_resample [B] float32 in [0,1)
 *   temperature   host float >= 0
 *   out_tokens    [B, K] int32 output: emitted tokens, then -1 padding
 *   num_emitted   [B] int32 output in [1, K]
 * Errors: INVALID_ARG (null, sizes < 1, temperature < 0 or not finite),
 *   UNSUPPORTED (K > 16, V > 1<<20).
 */
int clm_spec_verify(const float* target_logits, const float* draft_probs,
                    const int32_t* draft_tokens, const float* u_accept, const float* u_resample,
                    float temperature, int B, int K, int V, int32_t* out_tokens,
                    int32_t* num_emitted, hipStream_t stream);

/*
 * Speculative verification with a bonus token (Optimizing Streaming
 * Text-to-Speech Models ..., "Latency Benchmark Analysis": 0.28 target passes
 * per token at the acceptance rate 0.82 and K = 4 of "Speculative Decoding
 * for Acoustic Tokens", i.e. (1 - 0.82^5) / (1 - 0.82) = 3.50 tokens per
 * pass).  The target pass scores K + 1 positions: the K drafts and the one
 * after them.  Decisions for i = 0..K-1 are those of clm_spec_verify; if all
 * K drafts are accepted, one more token is drawn by inverse CDF at
 * u_resample[b] from softmax(target_logits[b,K,:] / T) (T = 0: its argmax).
 * At most one of the residual and bonus draws happens, so one uniform per
 * stream serves both.
 *   target_logits [B, K+1, V] float32,  draft_probs [B, K, V] float32
 *   draft_tokens  [B, K] int32 in [0, V)
 *   u_accept      [B, K] float32 in [0,1),  u_resample [B] float32 in [0,1)
 *   temperature   host float >= 0
 *   out_tokens    [B, K+1] int32 output: emitted tokens, then -1 padding
 *   num_emitted   [B] int32 output in [1, K+1]
 * Errors: as clm_spec_verify, with UNSUPPORTED for K + 1 > 16.
 */
int clm_spec_verify_bonus(const float* target_logits, const float* draft_probs,
                          const int32_t* draft_tokens, const float* u_accept, const float* u_resample,
                          float temperature, int B, int K, int V, int32_t* out_tokens,
                          int32_t* num_emitted, hipStream_t stream);


/* --------------------------------------------------------------------------
 * Multi-step decode loop as one HIP graph (How We Made a Text-to-Speech Model
 * Respond in Sub-50 ms, "Exploiting the regular building of the Code
 * Predictor": the whole frame-generation loop is captured as one graph;
 * section "Additional serving optimizations": graphs are kept for a set of
 * batch sizes; Optimizing Streaming Text-to-Speech Models ...,
 * "Engine-Level Optimizations with TensorRT-LLM": graph execution).
 * ------------------------------------------------------------------------ */

/*
 * Advance every stream's state by one step on the device:
 *     add = num_emitted ? num_emitted[b] (clamped to [0, T_new]) : T_new
 *     len_before[b] += add,  kv_len[b] += add,  positions[b, t] += add (t < T_new)
 * After speculative verification (num_emitted given) the next block of T_new
 * queries starts right after the kept tokens, overwriting the rejected
 * drafts' cache rows.  len_before, kv_len [B] int32 and positions [B, T_new]
 * int32 (NULL: none) are updated in place; num_emitted [B] int32 or NULL.
 * Errors: INVALID_ARG (null lengths, B or T_new < 1).
 */
int clm_advance_lengths(int32_t* len_before, int32_t* kv_len, int32_t* positions,
                        const int32_t* num_emitted, int B, int T_new, hipStream_t stream);

/*
 * One decode step per loop iteration, as the calls above would run it:
 *   append (rotary at logical positions when positions != NULL; the
 *   quantizing append when k_scale != NULL; both: the rotary FP8 append)
 *   -> attention (score scale
 *   1/sqrt(D); over the FP8 cache when k_scale != NULL) -> head (two
 *   layers with Mish when W2 != NULL) -> token
 *   choice (greedy, sampling or speculative verification) ->
 *   clm_advance_lengths.
 * Step s (0 <= s < n_steps) reads and writes slice s of each per-step array
 * (base + s * one step's elements).  All pointers are device memory owned by
 * the caller and must stay valid while the loop exists; the graph bakes them
 * in.  Sizes and meanings are those of the individual calls.
 */
typedef struct clm_decode_step_desc {
  int B, Kq, H_q, H_kv, D;          /* Kq queries (= rows appended) per stream and step */
  int block_size, num_blocks, max_blocks;
  int max_kv_len;                   /* bound on kv_len over all n_steps steps (split plan) */
  int G, V;                         /* head: G matrices [V, H_q*D] */
  clm_dtype dt;
  void* k_cache;                    /* paged pool, layout of clm_kv_cache_append */
  void* v_cache;
  const int32_t* block_table;       /* [B, max_blocks], must map every position the loop writes */
  int32_t* len_before;              /* [B]  advanced on the device after every step */
  int32_t* kv_len;                  /* [B]  (= len_before + Kq) advanced likewise */
  int32_t* positions;               /* [B, Kq] logical positions, or NULL for the plain append */
  float rope_base;                  /* used when positions != NULL */
  const void* k_new;                /* [n_steps][B, Kq, H_kv, D] */
  const void* v_new;                /* [n_steps][B, Kq, H_kv, D] */
  void* q;                          /* [n_steps][B, Kq, H_q, D] (rotated in place with positions) */
  const void* const* W;             /* host array of G device pointers, each [V, H_q*D] */
  const int32_t* head_id;           /* [B*Kq] or NULL when G == 1 */
  void* o;                          /* [n_steps][B, Kq, H_q, D] attention output (head input) */
  float* logits;                    /* [n_steps][B*Kq, V] */
  void* attn_workspace;             /* clm_decode_attention's workspace, or NULL: the library's */
  size_t attn_workspace_bytes;      /*   static scratch (clm_decode_attention_noalloc) */
  int mode;                         /* 0 greedy, 1 temperature sampling, 2 speculative verification,
                                       3 verification with a bonus token (clm_spec_verify_bonus): the
                                       Kq queries score the last kept token and Kd = Kq - 1 drafts */
  const float* temperature;         /* mode 1: [n_steps][B*Kq] */
  const float* uniforms;            /* mode 1: [n_steps][B*Kq] */
  int32_t* tokens;                  /* modes 0, 1: [n_steps][B*Kq] */
  float spec_temperature;           /* modes 2, 3 */
  const float* draft_probs;         /* modes 2, 3: [n_steps][B, Kd, V], Kd = Kq (mode 2) or Kq - 1 */
  const int32_t* draft_tokens;      /* modes 2, 3: [n_steps][B, Kd] */
  const float* u_accept;            /* modes 2, 3: [n_steps][B, Kd] */
  const float* u_resample;          /* modes 2, 3: [n_steps][B] */
  int32_t* out_tokens;              /* modes 2, 3: [n_steps][B, Kq] */
  int32_t* num_emitted;             /* modes 2, 3: [n_steps][B]; the lengths advance by these */
  float* k_scale;                   /* FP8 (E4M3) cache: the per-row key and value scales */
  float* v_scale;                   /*   [num_blocks, H_kv, block_size] of clm_kv_cache_append_fp8,
                                       with k_cache / v_cache in its byte layouts; both NULL for a
                                       cache of element type dt.  FP8 needs dt = CLM_BF16 and a
                                       caller attn_workspace (UNSUPPORTED otherwise); with positions
                                       the step appends by clm_rope_kv_cache_append_fp8 */
  const void* const* W2;            /* two-layer head (clm_codebook_head_mlp): host array of G
                                       device pointers, each [V, F]; W then holds the first layer,
                                       each [F, H_q*D].  NULL: the one-layer head */
  int F;                            /*   two-layer head: the widened size */
  void* act;                        /*   two-layer head: [B*Kq, F] bf16 activation scratch, reused
                                       by every step; bf16 only (UNSUPPORTED otherwise) */
} clm_decode_step_desc;

typedef struct clm_decode_loop clm_decode_loop;   /* opaque */

/*
 * Captures n_steps steps described by *desc (1 <= n_steps <= 1024) into one
 * HIP graph and instantiates it.  Host memory and the graph are allocated
 * here; no kernel runs.  Every argument is validated as the individual call
 * would validate it, before or during capture; on an error nothing is kept.
 * Checked mode must be off (it synchronises): UNSUPPORTED otherwise.
 * Errors: INVALID_ARG (null desc/loop, n_steps out of range, a null array the
 *   mode needs, mode not 0..3, mode 3 with Kq < 2, one FP8 scale array
 *   without the other, a two-layer head without act or with F < 1),
 *   UNSUPPORTED (an FP8 cache with dt other than CLM_BF16 or without
 *   attn_workspace; a two-layer head with dt other than CLM_BF16),
 *   the individual calls' errors, HIP.
 */
int clm_decode_loop_create(const clm_decode_step_desc* desc, int n_steps, clm_decode_loop** loop);

/* Runs the captured n_steps steps on `stream` (asynchronous).  Each launch
 * continues from the lengths the previous one left on the device. */
int clm_decode_loop_launch(clm_decode_loop* loop, hipStream_t stream);

/* Releases the graph (after the launches using it have completed). */
int clm_decode_loop_destroy(clm_decode_loop* loop);

/*
 * Host-only helper for a set of captured batch sizes: the index of the
 * smallest bucket_sizes[i] >= B (the first such on ties), or -1 if none.
 * A batch of B live streams runs in that bucket's loop with the remaining
 * slots padded by idle streams.
 */
int clm_pick_bucket(const int32_t* bucket_sizes, int n, int B);

#ifdef __cplusplus
}
#endif

#endif /* CLM_H */
