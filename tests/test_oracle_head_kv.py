"""Pins for the head and paged-append oracles (CPU only)."""

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
