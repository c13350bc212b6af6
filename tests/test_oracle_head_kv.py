"""Pins for the head and paged-append oracles (CPU only).

The two-layer head's Mish is pinned by the algebraic form
x * ((1+e^x)^2 - 1) / ((1+e^x)^2 + 1) (tanh(log y) = (y^2-1)/(y^2+1)), its
slope tanh(log 2) = 3/5 at zero, its asymptotes, and its minimum -0.30884
reported by Misra (2019); the layer structure by unit-vector and rank-one
weights."""

import numpy as np
import pytest

import oracle
import synth


def test_rank_one_weights_closed_form():
    # W = a b^T  ->  logits[r] = (h_r . b) a
    rng = np.random.default_rng(10)
    M, d, V = 5, 24, 40
    a, bvec = rng.standard_normal(V), rng.standard_normal(d)
    h = rng.standard_normal((M, d))
    logits = oracle.codebook_head(h, np.outer(a, bvec)[None])
    for r in range(M):
        np.testing.assert_allclose(logits[r], (h[r] @ bvec) * a, rtol=1e-12, atol=1e-12)


def test_unit_vector_rows_select_coordinates():
    # W[v] = e_{c(v)}  ->  logits[r, v] = h[r, c(v)]  (catches a transposed W)
    rng = np.random.default_rng(11)
    M, d, V = 3, 16, 50
    cols = rng.integers(0, d, size=V)
    W = np.zeros((1, V, d))
    W[0, np.arange(V), cols] = 1.0
    h = rng.standard_normal((M, d))
    np.testing.assert_array_equal(oracle.codebook_head(h, W), h[:, cols])


def test_grouped_heads_equal_separate_dense_calls():
    rng = np.random.default_rng(12)
    M, d, V, G = 9, 8, 12, 3
    W = rng.standard_normal((G, V, d))
    h = rng.standard_normal((M, d))
    hid = rng.integers(0, G, size=M)
    out = oracle.codebook_head(h, W, hid)
    for g in range(G):
        rows = np.nonzero(hid == g)[0]
        if rows.size:
            np.testing.assert_array_equal(out[rows], oracle.codebook_head(h[rows], W[g:g + 1]))
    with pytest.raises(ValueError):
        oracle.codebook_head(h, W, np.full(M, G))


def _mish_algebraic(x):
    # tanh(log y) = (y^2 - 1) / (y^2 + 1) with y = 1 + e^x: no tanh, no log
    y = 1.0 + np.exp(np.asarray(x, np.float64))
    return x * (y * y - 1.0) / (y * y + 1.0)


def test_mish_closed_forms():
    x = np.linspace(-8.0, 8.0, 161)
    np.testing.assert_allclose(oracle.mish(x), _mish_algebraic(x), rtol=1e-12, atol=1e-15)
    assert oracle.mish(0.0) == 0.0
    eps = 1e-8
    assert abs(oracle.mish(eps) / eps - 0.6) < 1e-7          # slope tanh(log 2) = 3/5
    assert abs(oracle.mish(40.0) - 40.0) < 1e-12             # ~ x for large x
    assert abs(oracle.mish(-40.0) - (-40.0 * np.exp(-40.0))) < 1e-25   # ~ x e^x for very negative x
    grid = np.linspace(-3.0, 0.0, 300001)
    m = oracle.mish(grid)
    assert abs(m.min() - (-0.30884)) < 1e-5 and abs(grid[np.argmin(m)] - (-1.1924)) < 1e-3


def test_bf16_rounding_of_the_activation():
    from oracle.head import round_to_bf16_f64
    vals = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -3.14159, 1e-30, 65504.5])
    r = round_to_bf16_f64(vals)
    # exactly representable: the low 16 bits of the float32 are zero
    assert np.all((r.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    # ties go to the even mantissa: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    assert r[0] == 1.0 and r[1] == 1.0 + 2 ** -6 and r[2] == 1.0
    assert abs(r[3] - -3.140625) == 0


def test_bf16_rounding_is_one_step_from_float64():
    """One rounding from the exact value: 1 + 2^-8 + 2^-30 lies above the
    midpoint between the bfloat16 neighbours 1 and 1 + 2^-7, so it rounds up;
    rounding to float32 first would land on the midpoint 1 + 2^-8 and then
    tie to 1.  Subnormal steps (2^-133), the largest finite value and the
    overflow threshold are the format's own."""
    from oracle.head import round_to_bf16_f64
    x = 1.0 + 2 ** -8 + 2 ** -30
    assert np.float32(x) == np.float32(1.0 + 2 ** -8)          # float32 first would tie ...
    assert round_to_bf16_f64(np.array([x]))[0] == 1.0 + 2 ** -7  # ... one step rounds up
    assert round_to_bf16_f64(np.array([-x]))[0] == -(1.0 + 2 ** -7)
    assert round_to_bf16_f64(np.array([2.0 ** -133 * 0.75]))[0] == 2.0 ** -133
    assert round_to_bf16_f64(np.array([2.0 ** -133 * 0.25]))[0] == 0.0
    assert round_to_bf16_f64(np.array([2.0 ** -126 * (1 + 2 ** -8)]))[0] == 2.0 ** -126  # tie to even
    top = (2 - 2 ** -7) * 2.0 ** 127                               # largest finite bfloat16
    assert round_to_bf16_f64(np.array([top]))[0] == top
    assert np.isinf(round_to_bf16_f64(np.array([(2 - 2 ** -9) * 2.0 ** 127])))[0]
    # away from midpoints, the same as the float32 -> bfloat16 rounding torch does
    import torch
    y = np.random.default_rng(3).standard_normal(20000) * 10.0 ** np.random.default_rng(4).integers(-30, 30, 20000)
    y32 = y.astype(np.float32).astype(np.float64)
    want = torch.from_numpy(y32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_to_bf16_f64(y32), want)


def test_two_layer_head_structure():
    # W1 rows = c_f e_{j(f)}: z[r, f] = c_f h[r, j(f)];  W2 = a b^T: logits = (act . b) a
    rng = np.random.default_rng(13)
    M, d, F, V = 6, 16, 24, 30
    h = rng.standard_normal((M, d))
    cols, c = rng.integers(0, d, size=F), rng.uniform(-3, 3, size=F)
    W1 = np.zeros((F, d))
    W1[np.arange(F), cols] = c
    a, bvec = rng.standard_normal(V), rng.standard_normal(F)
    act, logits = oracle.codebook_head_mlp(h, W1, np.outer(a, bvec), act_bf16=False)
    np.testing.assert_allclose(act, _mish_algebraic(c * h[:, cols]), rtol=1e-12, atol=1e-15)
    for r in range(M):
        np.testing.assert_allclose(logits[r], (act[r] @ bvec) * a, rtol=1e-12, atol=1e-12)
    act16, _ = oracle.codebook_head_mlp(h, W1, np.outer(a, bvec))
    assert np.all(np.abs(act16 - act) <= np.abs(act) * 2 ** -8 + 1e-38)   # half a bf16 ulp


def test_two_layer_grouped_heads_equal_separate_calls():
    rng = np.random.default_rng(14)
    M, d, F, V, G = 10, 8, 12, 9, 3
    W1, W2 = rng.standard_normal((G, F, d)), rng.standard_normal((G, V, F))
    h = rng.standard_normal((M, d))
    hid = rng.integers(0, G, size=M)
    act, logits = oracle.codebook_head_mlp(h, W1, W2, hid)
    for g in range(G):
        rows = np.nonzero(hid == g)[0]
        if rows.size:
            a_g, l_g = oracle.codebook_head_mlp(h[rows], W1[g], W2[g])
            np.testing.assert_array_equal(act[rows], a_g)
            np.testing.assert_array_equal(logits[rows], l_g)


def _small_step(cfg_index=3, B=6):
    return synth.make_inputs(cfg_index, B=B)


@pytest.mark.parametrize("cfg_index", [1, 4])
def test_append_then_gather_reproduces_logical_rows(cfg_index):
    x = _small_step(cfg_index, B=min(6, synth.get_config(cfg_index).B))
    bs = x.cfg.block_size
    k_pool, v_pool = x.build_pool(include_new=False)
    k2, v2 = oracle.kv_cache_append(k_pool, v_pool, x.block_table, x.len_before, x.k_new, x.v_new, bs)
    for b in range(x.cfg.B):
        K, V = oracle.gather_logical(k2, v2, x.block_table, b, int(x.kv_len[b]), bs)
        hist = slice(x.hist_off[b], x.hist_off[b + 1])
        np.testing.assert_array_equal(K, np.concatenate([x.k_hist[hist], x.k_new[b]]))
        np.testing.assert_array_equal(V, np.concatenate([x.v_hist[hist], x.v_new[b]]))


def test_append_touches_only_the_new_slots_and_splits_into_single_rows():
    x = synth.make_inputs(4, B=5)                       # 6 new rows per stream
    bs = x.cfg.block_size
    k_pool, v_pool = x.build_pool(include_new=False)
    k_all, v_all = oracle.kv_cache_append(k_pool, v_pool, x.block_table, x.len_before, x.k_new, x.v_new, bs)
    # T appends of one row == one append of T rows (bit-exact)
    k1, v1 = k_pool, v_pool
    for t in range(x.cfg.Kq):
        k1, v1 = oracle.kv_cache_append(k1, v1, x.block_table, x.len_before + t,
                                        x.k_new[:, t:t + 1], x.v_new[:, t:t + 1], bs)
    np.testing.assert_array_equal(k1, k_all)
    np.testing.assert_array_equal(v1, v_all)
    # exactly B*T*H*D elements changed in each pool (NaN -> finite)
    changed_k = np.count_nonzero(k_all.view(np.uint16) != k_pool.view(np.uint16))
    changed_v = np.count_nonzero(v_all.view(np.uint16) != v_pool.view(np.uint16))
    n = x.cfg.B * x.cfg.Kq * x.cfg.H_kv * x.cfg.D
    assert changed_k == n and changed_v == n
    # and the pool built with the new rows matches
    kp, vp = x.build_pool(include_new=True)
    np.testing.assert_array_equal(kp, k_all)
    np.testing.assert_array_equal(vp, v_all)
