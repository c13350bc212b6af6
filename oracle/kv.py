"""Oracle: appending a step's new K/V rows into the paged KV cache.

Test infrastructure only (see the package docstring).

Optimizing Streaming Text-to-Speech Models ..., "Dynamic Token-Level
Batching": the cache is a static pool cut into fixed 16-token blocks that
requests take from a global free list.  A stream's token at position p lives
in block ``block_table[b, p // bs]`` at slot ``p % bs``.  Layout of one
block (per KV head): keys as [bs, D] rows, values transposed as [D, bs].

Appending writes rows t = 0..T_new-1 of stream b at positions
len_before[b] + t and leaves every other slot untouched.
"""

from __future__ import annotations

import numpy as np


def kv_cache_append(k_pool, v_pool, block_table, len_before, k_new, v_new, block_size):
    """Returns updated copies of (k_pool, v_pool).
    k_pool [nb, H, bs, D], v_pool [nb, H, D, bs], k_new/v_new [B, T, H, D]."""
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    B, T = k_new.shape[0], k_new.shape[1]
    for b in range(B):
        for t in range(T):
            pos = int(len_before[b]) + t
            blk = int(block_table[b, pos // block_size])
            slot = pos % block_size
            k[blk, :, slot, :] = k_new[b, t]
            v[blk, :, :, slot] = v_new[b, t]
    return k, v


def gather_logical(k_pool, v_pool, block_table, b, n, block_size):
    """Read stream b's first n positions back out of the pool as
    K, V [n, H, D] (same element type as the pool)."""
    H, D = k_pool.shape[1], k_pool.shape[3]
    K = np.empty((n, H, D), k_pool.dtype)
    V = np.empty((n, H, D), v_pool.dtype)
    for pos in range(n):
        blk = int(block_table[b, pos // block_size])
        slot = pos % block_size
        K[pos] = k_pool[blk, :, slot, :]
        V[pos] = v_pool[blk, :, :, slot]
    return K, V
