"""Oracle: rotary position embedding at logical positions (float64).

Test infrastructure only (see the package docstring).

TontaubeV1 (Section 3.3 layout paragraph and the vLLM-adapter paragraph):
positions are logical coordinates, not physical sequence indices; rotary
attention depends only on coordinate differences, so the adapters add one
uniform constant to every prefill coordinate and decode stays
identity-indexed.  The speculative-decoding blog (section "Engine-Level
Optimizations with TensorRT-LLM", kernel-fusion item) fuses the rotary
embedding with the key-value cache write.

A vector x of even width D at position p is rotated pairwise:

  theta_i = base ** (-2 i / D),   a_i = p * theta_i,   i = 0 .. D/2 - 1
  (x_i, x_{i+D/2})  ->  (x_i cos a_i - x_{i+D/2} sin a_i,
                         x_i sin a_i + x_{i+D/2} cos a_i)

Readings where the pages leave a step open: the pairing is the half-split
one (dimension i with i + D/2) used by the vLLM decode path the pages name,
the whole head width is rotated, and the base is a caller argument.  In the
fused append, the step's queries and new keys take the logical positions
supplied for the step's new tokens (the K-query block's queries are the K
appended tokens); values are not rotated.
"""

from __future__ import annotations

import numpy as np

from .kv import kv_cache_append


def rope(x, pos, base):
    """x [..., D] (any float type) rotated at integer positions pos
    (broadcast against x[..., 0]); returns float64."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    if D % 2:
        raise ValueError("rotary width must be even")
    half = D // 2
    theta = np.float64(base) ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    a = np.asarray(pos, np.float64)[..., None] * theta
    c, s = np.cos(a), np.sin(a)
    x0, x1 = x[..., :half], x[..., half:]
    return np.concatenate([x0 * c - x1 * s, x0 * s + x1 * c], axis=-1)


def rope_kv_cache_append(q, k_pool, v_pool, block_table, len_before, positions, k_new, v_new,
                         block_size, base):
    """q [B, T, H_q, D]; k_new, v_new [B, T, H_kv, D]; positions [B, T] logical.
    Returns (q rotated [B, T, H_q, D] float64, k_pool, v_pool) with the
    rotated keys and the plain values written at slots len_before[b] + t."""
    pos = np.asarray(positions, np.int64)
    q_rot = rope(q, pos[:, :, None], base)
    k_rot = rope(k_new, pos[:, :, None], base)
    k, v = kv_cache_append(np.asarray(k_pool, np.float64), v_pool, block_table, len_before, k_rot, v_new,
                           block_size)
    return q_rot, k, v
