"""Pins for the FP8 (E4M3) KV-cache oracle (CPU only).

E4M3's defining values (1.0 = 0x38, the largest 448 = 0x7E, the smallest
normal 2^-6 = 0x08 and subnormal 2^-9 = 0x01, NaN = 0x7F), a brute-force
nearest-value search over all 254 finite codes with ties to the even code,
the half-step error bound of a scaled row, and the attention oracle on
dequantized rows equal to the plain oracle when the rows are exactly
representable.
"""

import numpy as np

import oracle
import synth
from oracle import fp8


def test_defining_values():
    d = fp8.e4m3_decode
    assert d(0x38) == 1.0 and d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6 and d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x3C) == 1.5 and d(0x40) == 2.0 and d(0x77) == 240.0


def test_every_finite_code_round_trips_and_order_is_value_order():
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8.e4m3_decode(codes)
    ok = ~np.isnan(vals)
    np.testing.assert_array_equal(fp8.e4m3_encode(vals[ok]), codes[ok])
    pos = vals[:128][~np.isnan(vals[:128])]
    assert np.all(np.diff(pos) > 0)


def test_encode_is_the_nearest_value_with_ties_to_even_by_brute_force():
    rng = np.random.default_rng(3)
    codes = np.arange(128, dtype=np.uint8)
    vals = fp8.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    cand_c, cand_v = codes[fin], vals[fin]
    # random points plus every exact midpoint between neighbours
    mids = (cand_v[1:] + cand_v[:-1]) / 2
    xs = np.concatenate([rng.uniform(0, 448, 3000), mids, cand_v])
    got = fp8.e4m3_encode(xs)
    for x, g in zip(xs, got):
        dist = np.abs(cand_v - x)
        best = np.nonzero(dist == dist.min())[0]
        want = cand_c[best[0]] if len(best) == 1 else [c for c in cand_c[best] if c % 2 == 0][0]
        assert g == want, (x, g, want)
    # sign: the magnitude's code with bit 7 set
    np.testing.assert_array_equal(fp8.e4m3_encode(-xs[:100]), got[:100] | 0x80)


def test_row_quantization_error_is_within_half_a_step():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 128)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    codes, scale = fp8.quantize_rows(x)
    y = fp8.dequantize_rows(codes, scale)
    # the largest magnitude of each row maps to +-448 (code 0x7E)
    assert np.all((codes & 0x7F).max(axis=1) == 0x7E)
    # error <= half the spacing at that magnitude: 2^-4 relative for normals
    # (3 mantissa bits), 2^-10 * scale absolute in the subnormal range
    err = np.abs(y - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)
    z_codes, z_scale = fp8.quantize_rows(np.zeros((2, 8), np.float32))
    assert np.all(z_scale == 1.0) and np.all((z_codes & 0x7F) == 0)


def test_fp8_append_and_attention_on_exactly_representable_rows():
    # rows made of E4M3 values times a power of two with 448 in every row
    # quantize without error, so fp8 attention equals the plain oracle
    x = synth.make_inputs(2, B=3)
    c = x.cfg
    rng = np.random.default_rng(5)
    vals = fp8.e4m3_decode(np.arange(0x00, 0x7E, dtype=np.uint8))
    def exact(shape):
        a = rng.choice(vals, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        a[..., 0] = 448.0
        return (a / 64.0).astype(np.float32)
    nb = x.block_table.max() + 1
    kp = np.zeros((nb, c.H_kv, c.D // 8, c.block_size, 8), np.uint8)
    vp = np.zeros((nb, c.H_kv, c.D, c.block_size), np.uint8)
    ks = np.ones((nb, c.H_kv, c.block_size), np.float32)
    vs = np.ones((nb, c.H_kv, c.block_size), np.float32)
    n = int(x.kv_len.max())
    K_all = exact((c.B, n, c.H_kv, c.D))
    V_all = exact((c.B, n, c.H_kv, c.D))
    zero = np.zeros(c.B, np.int32)
    kp, vp, ks, vs = fp8.fp8_kv_cache_append(kp, vp, ks, vs, x.block_table, zero, K_all, V_all, c.block_size)
    keys, vals_ = [], []
    for b in range(c.B):
        K, V = fp8.gather_dequantized(kp, vp, ks, vs, x.block_table, b, int(x.kv_len[b]), c.block_size)
        np.testing.assert_array_equal(K, K_all[b, :int(x.kv_len[b])])
        np.testing.assert_array_equal(V, V_all[b, :int(x.kv_len[b])])
        keys.append(K)
        vals_.append(V)
    q = synth.bf16_bits_to_f32(x.q)
    got = oracle.decode_attention(q, keys, vals_, x.kv_len, 1 / np.sqrt(c.D), c.H_kv)
    want = oracle.decode_attention(q, [K_all[b, :int(x.kv_len[b])] for b in range(c.B)],
                                   [V_all[b, :int(x.kv_len[b])] for b in range(c.B)], x.kv_len,
                                   1 / np.sqrt(c.D), c.H_kv)
    np.testing.assert_array_equal(got, want)
