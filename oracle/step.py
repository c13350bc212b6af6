"""Oracle: one whole decode step, chained.

Test infrastructure only (see the package docstring).

TTS Serving, in depth ("Token generation under a frame budget"): a decode
step appends the new frame's K/V to the cache, attends over the cache, and
turns the result into the next token.  Here, per stream b:

  1. append the step's Kq new K/V rows             (kv.kv_cache_append)
  2. o = decode attention of the Kq queries         (attention.decode_attention)
  3. o is delivered in the step's element type: rounded to bfloat16 (nearest,
     ties to even) for bf16 steps, kept float32 for f32 steps
  4. h = o flattened to [B*Kq, H_q*D] (order b, j, head, dim)
  5. logits = codebook head of h, as float32       (head.codebook_head)
  6. greedy / sampled token per row, or speculative verification of the
     K drafted tokens of each stream               (sampling, verify)
Inputs are logical per-stream K/V lists; the paged pool is not involved
except in step 1, which the caller checks separately.
"""

from __future__ import annotations

import numpy as np

from .attention import decode_attention
from .head import codebook_head
from .sampling import sample_or_argmax
from .verify import spec_verify


def round_to_bf16(x) -> np.ndarray:
    """float -> nearest bfloat16 value (ties to even), returned as float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    return np.where(np.isnan(f), np.float32(np.nan), out)


def decode_step(q, keys, values, kv_len, scale, n_kv_heads, W, head_id, elem_bf16,
                mode="greedy", temperature=None, uniforms=None, spec=None, streams=None):
    """Steps 2-6 above.  Returns dict with o (float64), h (float32 values fed
    to the head), logits (float32) and tokens or (out_tokens, num_emitted).
    ``streams`` restricts the work to a subset of streams."""
    B, Kq, Hq, D = q.shape
    o = decode_attention(q, keys, values, kv_len, scale, n_kv_heads, streams=streams)
    o_dt = round_to_bf16(o) if elem_bf16 else o.astype(np.float32)
    h = o_dt.reshape(B * Kq, Hq * D)
    rows = None if streams is None else [b * Kq + j for b in streams for j in range(Kq)]
    logits = codebook_head(h, W, head_id, rows=rows).astype(np.float32)
    out = dict(o=o, h=h, logits=logits, rows=rows)
    sel = np.arange(B * Kq) if rows is None else np.array(rows)
    if mode == "spec":
        V = logits.shape[1]
        toks, num = spec_verify(logits.reshape(B, Kq, V), spec["draft_probs"], spec["draft_tokens"],
                                spec["u_accept"], spec["u_resample"], float(temperature), streams=streams)
        out.update(out_tokens=toks, num_emitted=num)
    else:
        tok = np.full(B * Kq, -1, np.int32)
        temp = None if temperature is None else np.asarray(temperature, np.float32)[sel]
        uni = None if uniforms is None else np.asarray(uniforms, np.float32)[sel]
        tok[sel] = sample_or_argmax(logits[sel], temp, uni)
        out.update(tokens=tok)
    return out
