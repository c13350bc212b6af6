"""Pins for the rotary-embedding oracle (CPU only).

The property the pages rely on - rotary attention depends only on coordinate
differences, so adding one constant to every coordinate changes no score
(TontaubeV1, vLLM-adapter paragraph) - plus closed forms: position 0 is the
identity, D = 2 is a plane rotation by p radians, each pair keeps its norm,
and theta_i = base^(-2i/D) shows in the pair rotated by exactly p*theta_i.
"""

import numpy as np

import oracle
import synth


def test_position_zero_and_plane_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 8))
    np.testing.assert_array_equal(oracle.rope(x, 0, 10000.0), x)
    # D = 2: theta_0 = 1, a plane rotation by p radians
    v = np.array([0.6, -0.8])
    for p in (1, 7, 1000):
        c, s = np.cos(p), np.sin(p)
        np.testing.assert_allclose(oracle.rope(v, p, 10000.0), [0.6 * c + 0.8 * s, 0.6 * s - 0.8 * c],
                                   rtol=0, atol=1e-12)


def test_pairs_keep_their_norm_and_frequencies_follow_the_base():
    rng = np.random.default_rng(2)
    D, base = 16, 500.0
    x = rng.standard_normal(D)
    y = oracle.rope(x, 37, base)
    half = D // 2
    np.testing.assert_allclose(np.hypot(y[:half], y[half:]), np.hypot(x[:half], x[half:]), rtol=1e-12)
    # a unit vector in dimension i turns by 37 * base^(-2i/D) exactly
    for i in range(half):
        e = np.zeros(D)
        e[i] = 1.0
        r = oracle.rope(e, 37, base)
        ang = np.arctan2(r[i + half], r[i])
        want = np.angle(np.exp(1j * 37 * base ** (-2.0 * i / D)))
        assert abs(ang - want) < 1e-9


def test_scores_depend_only_on_the_position_difference():
    rng = np.random.default_rng(3)
    D, base = 128, 1.0e6
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for m, n in ((5, 3), (700, 12), (9000, 8999)):
        s0 = oracle.rope(q, m, base) @ oracle.rope(k, n, base)
        np.testing.assert_allclose(s0, oracle.rope(q, m - n, base) @ k, rtol=1e-9, atol=1e-9)
        # one uniform constant added to every coordinate changes no score
        for c in (1, 250, 123456):
            np.testing.assert_allclose(oracle.rope(q, m + c, base) @ oracle.rope(k, n + c, base), s0,
                                       rtol=1e-9, atol=1e-9)


def test_fused_append_writes_rotated_keys_and_plain_values():
    x = synth.make_inputs(2, B=3)
    c = x.cfg
    kp, vp = x.build_pool(include_new=False)
    kp, vp = synth.bf16_bits_to_f32(kp), synth.bf16_bits_to_f32(vp)
    pos = (x.len_before[:, None] + 1000 + np.arange(c.Kq)[None, :]).astype(np.int32)
    q = synth.bf16_bits_to_f32(x.q)
    kn, vn = synth.bf16_bits_to_f32(x.k_new), synth.bf16_bits_to_f32(x.v_new)
    q_rot, k2, v2 = oracle.rope_kv_cache_append(q, kp, vp, x.block_table, x.len_before, pos, kn, vn,
                                               c.block_size, 1.0e6)
    k_plain, v_plain = oracle.kv_cache_append(kp.astype(np.float64), vp, x.block_table, x.len_before,
                                              oracle.rope(kn, pos[:, :, None], 1.0e6), vn, c.block_size)
    np.testing.assert_array_equal(k2, k_plain)
    np.testing.assert_array_equal(v2, v_plain)
    np.testing.assert_allclose(q_rot, oracle.rope(q, pos[:, :, None], 1.0e6), rtol=0, atol=0)
    # values untouched by the rotation; norms of q pairs kept
    half = c.D // 2
    np.testing.assert_allclose(np.hypot(q_rot[..., :half], q_rot[..., half:]),
                               np.hypot(q[..., :half], q[..., half:]), rtol=1e-6)
