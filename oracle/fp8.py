"""Oracle: FP8 (E4M3) key/value cache with one scale per cached row.

Test infrastructure only (see the package docstring).

The speculative-decoding blog (section "Engine-Level Optimizations with
TensorRT-LLM", FP8 item) applies FP8 quantization to the target model's
attention; here it is taken to the KV cache, which every decode step reads.

E4M3 (the OCP 8-bit float with 4 exponent bits, bias 7, 3 mantissa bits, no
infinities; 0x7F / 0xFF are NaN): normal values (-1)^s 2^(e-7) (1 + m/8) for
e = 1..15 (with e = 15, m = 7 reserved for NaN, so the largest is 448);
subnormals (-1)^s 2^-6 (m/8) for e = 0.

A row x (one token's D values of one KV head) is stored as
  scale = max|x| / 448            (1 when the row is all zero)
  code_i = E4M3( x_i / scale )    round to nearest, ties to even
and read back as decode(code_i) * scale.  Cache layout: keys as 8-dimension
groups, k_pool[block, head, d // 8, slot, d % 8] (each group of a block's
keys contiguous), values transposed as in the bf16 cache, v_pool[block,
head, d, slot].  Readings where the page leaves a step open: the E4M3 variant, one fp32 scale per (token, KV head) row for keys
and for values, the scale and the division in float32, and the quotient
clamped to +-448 before rounding.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def _all_finite_values():
    codes = np.arange(128, dtype=np.uint8)
    vals = e4m3_decode(codes)
    keep = ~np.isnan(vals)
    return codes[keep], vals[keep]


_POS_CODES, _POS_VALS = _all_finite_values()          # ascending: code order is value order


def e4m3_encode(x):
    """float values (|x| <= 448) -> uint8 codes, round to nearest with ties to
    the even code (the one whose lowest mantissa bit is 0); the sign bit
    follows x's sign, so -0 and negative values that round to 0 give 0x80."""
    x = np.asarray(x, np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3_encode: value outside [-448, 448]")
    a = np.abs(x)
    hi = np.searchsorted(_POS_VALS, a, side="left")       # first value >= a
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    vlo, vhi = _POS_VALS[lo], _POS_VALS[hi]
    dlo, dhi = a - vlo, vhi - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0) & (hi != lo))
    pick_hi |= (vhi == a)
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    # the sign bit is x's sign bit, also when the magnitude rounds to zero
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def quantize_rows(x):
    """x [..., D] (float32 values) -> (codes [..., D] uint8, scale [...] float32)."""
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0)).astype(np.float32)
    q = (x / scale[..., None]).astype(np.float32)
    q = np.clip(q, -E4M3_MAX, E4M3_MAX)
    return e4m3_encode(q), scale


def dequantize_rows(codes, scale):
    return e4m3_decode(codes) * np.asarray(scale, np.float64)[..., None]


def fp8_kv_cache_append(k_pool, v_pool, k_scale, v_scale, block_table, len_before, k_new, v_new,
                        block_size):
    """Quantize the new rows and write them into copies of the fp8 pool:
    k_pool [nb, H, D/8, bs, 8] uint8, v_pool [nb, H, D, bs] uint8, k_scale
    and v_scale [nb, H, bs] float32; k_new, v_new [B, T, H, D] (float32
    values)."""
    k, v = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    ks, vs = np.array(k_scale, copy=True), np.array(v_scale, copy=True)
    kq, kscale = quantize_rows(k_new)
    vq, vscale = quantize_rows(v_new)
    B, T = k_new.shape[0], k_new.shape[1]
    for b in range(B):
        for t in range(T):
            pos = int(len_before[b]) + t
            blk = int(block_table[b, pos // block_size])
            slot = pos % block_size
            k[blk, :, :, slot, :] = kq[b, t].reshape(kq.shape[2], -1, 8)
            v[blk, :, :, slot] = vq[b, t]
            ks[blk, :, slot] = kscale[b, t]
            vs[blk, :, slot] = vscale[b, t]
    return k, v, ks, vs


def gather_dequantized(k_pool, v_pool, k_scale, v_scale, block_table, b, n, block_size):
    """Stream b's first n positions as dequantized K, V [n, H, D] float64."""
    H, D = k_pool.shape[1], k_pool.shape[2] * k_pool.shape[4]
    K = np.empty((n, H, D))
    V = np.empty((n, H, D))
    for pos in range(n):
        blk = int(block_table[b, pos // block_size])
        slot = pos % block_size
        K[pos] = dequantize_rows(k_pool[blk, :, :, slot, :].reshape(H, D), k_scale[blk, :, slot])
        V[pos] = dequantize_rows(v_pool[blk, :, :, slot], v_scale[blk, :, slot])
    return K, V
