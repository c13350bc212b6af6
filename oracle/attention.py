"""Oracle: decode attention over each stream's logical KV cache (float64).

Test infrastructure only (see the package docstring).

Definition (TTS Serving, in depth, "Token generation under a frame budget":
each decode step attends from the new frame's query over the stream's KV
cache; Optimizing Streaming Text-to-Speech Models ..., "Speculative Decoding
for Acoustic Tokens": one target pass scores K drafted positions, which is a
causal block of K queries):

  for stream b, query j in [0, Kq), query head h:
      n   = kv_len[b] - (Kq - 1 - j)        keys visible to query j
      g   = h // (H_q / H_kv)               its KV head (consecutive query
                                            heads share one KV head)
      w   = softmax(scale * K[0:n, g] . q)  over the n visible keys
      o   = sum_t w[t] * V[t, g]

Readings where the pages are silent: the scale is passed in (1/sqrt(D) by
default); ``kv_len`` counts the keys the last query sees, including the rows
appended this step; q and k arrive already position-rotated.
"""

from __future__ import annotations

import numpy as np


def attention_weights(q_vec, k_rows, scale):
    """Softmax weights of one query over the rows of ``k_rows`` [n, D]."""
    s = scale * (np.asarray(k_rows, np.float64) @ np.asarray(q_vec, np.float64))
    e = np.exp(s - s.max())
    return e / e.sum()


def attend(q_vec, k_rows, v_rows, scale):
    """One query head over n keys: sum_t w[t] * v_rows[t]."""
    w = attention_weights(q_vec, k_rows, scale)
    return w @ np.asarray(v_rows, np.float64)


def decode_attention(q, keys, values, kv_len, scale, n_kv_heads, streams=None):
    """q [B, Kq, H_q, D]; keys[b], values[b] are [kv_len[b], H_kv, D] arrays
    (index with the stream number); returns o [B, Kq, H_q, D] float64.
    ``streams`` restricts the work to a subset (other rows stay zero)."""
    q = np.asarray(q, np.float64)
    B, Kq, Hq, D = q.shape
    if Hq % n_kv_heads:
        raise ValueError("H_q must be a multiple of H_kv")
    group = Hq // n_kv_heads
    out = np.zeros((B, Kq, Hq, D), np.float64)
    for b in (range(B) if streams is None else streams):
        K = np.asarray(keys[b], np.float64)
        V = np.asarray(values[b], np.float64)
        if K.shape[0] != kv_len[b]:
            raise ValueError("stream %d: %d key rows for kv_len %d" % (b, K.shape[0], kv_len[b]))
        for j in range(Kq):
            n = int(kv_len[b]) - (Kq - 1 - j)
            if n < 1:
                raise ValueError("query %d of stream %d sees no key" % (j, b))
            for h in range(Hq):
                g = h // group
                out[b, j, h] = attend(q[b, j, h], K[:n, g, :], V[:n, g, :], scale)
    return out
