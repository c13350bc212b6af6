// Launch plans: the host-side arithmetic that sizes the attention split plan
// and the head's tiles.  Deterministic functions of the call's sizes, shared
// by the workspace queries and the launches (kept apart from the kernel
// sources so a host-only build, e.g. with sanitizers, can use them).
#include <cstddef>

#include "clm_launch.h"

namespace clm {
namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kHeadWorkgroups = 256;   // workgroups the head's tile choice aims for
constexpr int kXcdCount = 8;           // the head pads its tile rows to whole XCD rounds

}  // namespace

bool plan_decode_attention(int B, int Kq, int H_q, int H_kv, int D, int max_kv_len, AttnPlan* p) {
  if (B < 1 || Kq < 1 || H_kv < 1 || H_q % H_kv || max_kv_len < 1) return false;
  const int nr = (H_q / H_kv) * Kq;
  if (nr > 16) return false;
  p->nr = nr;
  p->nr_tmpl = nr <= 1 ? 1 : nr <= 2 ? 2 : nr <= 4 ? 4 : nr <= 8 ? 8 : nr <= 12 ? 12 : 16;
  // Split length, taking lengths to average half the maximum (est = expected
  // token-heads).  Long splits cost less per token (fewer partial results,
  // fewer pipeline restarts); short ones keep small batches spread over the
  // CUs.  An item spans at most 64 blocks of 16 tokens (one block id per lane).
  // 1-2 query rows (vector kernel; FP8 matrix-core kernel): the largest power
  // of two <= est / 512, clamped to [64, 1024].  Measured on MI355X: 256
  // streams x log-uniform 64..8192 keys run 8% faster at 1024 than at 256
  // tokens, 64 streams x 200..3000 keys 25% faster at 512-1024, 16 streams x
  // 100..1500 keys best at 128.
  // 3-16 rows (matrix-core kernel, whose tiles cost more per token): the
  // smallest of 64, 128, 192, 256, 384, 512 at or above est / 768 (about 768
  // items for the chip).  The coarse steps keep a plan over a range of batch
  // sizes, so compacting a batch leaves results bit-identical more often
  // (384 tokens from 26 to 37 streams of up to ~2000 keys).  Blocks of 6
  // queries, bf16 and FP8 caches, against the earlier power-of-two rule
  // (est / 256): 32 streams x 300..2000 keys 384 tokens, 35.1 against 36.0 us
  // (FP8 27.6 against 32.2); 32 x 100..800 keys 192 tokens, 22.5 against
  // 24.5 us (FP8 20.3 against 22.4); 16 x 300..2000 keys 192 tokens, 24.2
  // against 24.7 us (FP8 20.2 against 22.4); 8, 64 and 128 streams and 32 x
  // 2000..8000 keys keep their split.  1024 tokens took 59.8 against 39.9 us
  // at 512 for 32 x 300..2000 keys.
  const double est = (double)B * H_kv * (max_kv_len > 1 ? max_kv_len / 2.0 : 1.0);
  long split = 64;
  if (nr > 2) {
    const double want = est / 768.0;
    split = 512;
    for (int c : {64, 128, 192, 256, 384})
      if ((double)c >= want) { split = c; break; }
  } else {
    while (split < 1024 && (double)(split * 2) * 512.0 <= est) split *= 2;
  }
  p->split = (int)split;
  p->max_splits = (int)((max_kv_len + split - 1) / split);
  const size_t slots = (size_t)B * H_kv * p->max_splits * p->nr_tmpl;
  p->ml_offset = 0;
  p->acc_offset = p->ml_offset + align256(slots * 2 * sizeof(float));
  p->total_bytes = p->acc_offset + align256(slots * (size_t)D * sizeof(float));
  return true;
}

HeadPlan plan_codebook_head(int M, int V, int G) {
  // MR in {32, 64, 96, 128}: the fewest padded rows for the rows one stage
  // is expected to hold (all M for one stage; M/G on average otherwise), the
  // larger on ties; NV in {128, 64, 32}: the widest that still gives
  // kHeadWorkgroups working workgroups; 8 waves where the tile is tall enough to
  // keep two waves per SIMD busy (and its rows split into 64-row DMA rounds).
  HeadPlan p{};
  const int m_est = G == 1 ? M : (M + G - 1) / G;
  int mr = 128;
  for (int c : {96, 64, 32})
    if ((m_est + c - 1) / c * c < (m_est + mr - 1) / mr * mr) mr = c;
  const int rc_est = (m_est + mr - 1) / mr;
  int nv = 32;
  for (int c : {128, 64})
    if ((long)((V + c - 1) / c) * rc_est * G >= kHeadWorkgroups) { nv = c; break; }
  p.mr = mr;
  p.nv = nv;
  p.nw = (mr >= 96 && (nv + mr) % 64 == 0) ? 8 : 4;
  p.row_chunks = (M + mr - 1) / mr;
  p.nvt = (V + nv - 1) / nv;
  p.nvt_pad = (p.nvt + kXcdCount - 1) / kXcdCount * kXcdCount;
  p.workspace_bytes = 0;
  return p;
}

}  // namespace clm
