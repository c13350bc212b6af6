"""Pins for the attention oracle: closed forms and invariants (CPU only)."""

import math

import numpy as np
import pytest

import oracle


def _rng(seed=0):
    return np.random.default_rng(seed)


def test_equal_keys_give_mean_of_visible_values_causal_block():
    # All keys equal -> every weight is 1/n, so o_j = mean of the first n_j
    # value rows; with a 4-query causal block n_j = kv_len - (Kq-1-j).
    rng = _rng(1)
    B, Kq, Hq, Hk, D = 2, 4, 4, 2, 8
    kv_len = np.array([7, 12])
    keys = [np.broadcast_to(rng.standard_normal((1, Hk, D)), (n, Hk, D)).copy() for n in kv_len]
    vals = [rng.standard_normal((n, Hk, D)) for n in kv_len]
    q = rng.standard_normal((B, Kq, Hq, D))
    o = oracle.decode_attention(q, keys, vals, kv_len, 1 / math.sqrt(D), Hk)
    for b in range(B):
        for j in range(Kq):
            n = kv_len[b] - (Kq - 1 - j)
            for h in range(Hq):
                expect = vals[b][:n, h // (Hq // Hk)].mean(axis=0)
                np.testing.assert_allclose(o[b, j, h], expect, rtol=1e-12, atol=1e-12)


def test_two_keys_logistic_closed_form():
    # n = 2: w0 = 1 / (1 + exp(scale * (s1 - s0))) with s_t = q.k_t.
    rng = _rng(2)
    D = 16
    q = rng.standard_normal(D)
    k = rng.standard_normal((2, D))
    scale = 0.3
    w = oracle.attention_weights(q, k, scale)
    s0, s1 = float(k[0] @ q), float(k[1] @ q)
    w0 = 1.0 / (1.0 + math.exp(scale * (s1 - s0)))
    assert w[0] == pytest.approx(w0, rel=1e-12)
    assert w[1] == pytest.approx(1 - w0, rel=1e-12)


def test_weights_sum_to_one_and_one_hot_values_return_weights():
    rng = _rng(3)
    n, D = 9, 12
    q = rng.standard_normal(D)
    k = rng.standard_normal((n, D))
    w = oracle.attention_weights(q, k, 0.25)
    assert abs(w.sum() - 1.0) < 1e-12
    assert np.all(w > 0)
    v = np.eye(n, D)                       # V_t = e_t (D >= n)
    o = oracle.attend(q, k, v, 0.25)
    np.testing.assert_allclose(o[:n], w, rtol=1e-12)
    np.testing.assert_allclose(o[n:], 0.0)


def test_single_key_and_dominant_key():
    rng = _rng(4)
    D = 32
    q = rng.standard_normal(D)
    k = rng.standard_normal((1, D))
    v = rng.standard_normal((1, D))
    np.testing.assert_allclose(oracle.attend(q, k, v, 0.1), v[0], rtol=1e-12)
    k = rng.standard_normal((20, D)) * 0.01
    k[13] = q * 10.0                        # q.k_13 dwarfs the others
    v = rng.standard_normal((20, D))
    np.testing.assert_allclose(oracle.attend(q, k, v, 1.0), v[13], rtol=1e-9, atol=1e-9)


def test_permuting_kv_pairs_and_batch_order_is_invariant():
    rng = _rng(5)
    B, Hq, Hk, D = 3, 4, 2, 8
    kv_len = np.array([5, 9, 3])
    keys = [rng.standard_normal((n, Hk, D)) for n in kv_len]
    vals = [rng.standard_normal((n, Hk, D)) for n in kv_len]
    q = rng.standard_normal((B, 1, Hq, D))
    o = oracle.decode_attention(q, keys, vals, kv_len, 0.35, Hk)
    perm = [rng.permutation(n) for n in kv_len]
    o2 = oracle.decode_attention(q, [k[p] for k, p in zip(keys, perm)],
                                 [v[p] for v, p in zip(vals, perm)], kv_len, 0.35, Hk)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-14)
    bp = np.array([2, 0, 1])
    o3 = oracle.decode_attention(q[bp], [keys[i] for i in bp], [vals[i] for i in bp], kv_len[bp], 0.35, Hk)
    np.testing.assert_allclose(o3, o[bp], rtol=0, atol=0)


def test_gqa_equals_mha_with_repeated_kv_heads():
    # Query heads 2g and 2g+1 share KV head g (consecutive grouping).
    rng = _rng(6)
    B, Kq, Hq, Hk, D = 2, 3, 8, 2, 8
    kv_len = np.array([6, 10])
    keys = [rng.standard_normal((n, Hk, D)) for n in kv_len]
    vals = [rng.standard_normal((n, Hk, D)) for n in kv_len]
    q = rng.standard_normal((B, Kq, Hq, D))
    o = oracle.decode_attention(q, keys, vals, kv_len, 0.2, Hk)
    rep = Hq // Hk
    o_mha = oracle.decode_attention(q, [np.repeat(k, rep, axis=1) for k in keys],
                                    [np.repeat(v, rep, axis=1) for v in vals], kv_len, 0.2, Hq)
    np.testing.assert_allclose(o, o_mha, rtol=1e-12, atol=1e-14)
    # the other plausible grouping (h -> h % H_kv, i.e. tiled heads) differs
    o_tiled = oracle.decode_attention(q, [np.tile(k, (1, rep, 1)) for k in keys],
                                      [np.tile(v, (1, rep, 1)) for v in vals], kv_len, 0.2, Hq)
    assert not np.allclose(o, o_tiled)


def test_causal_block_ignores_keys_beyond_each_query():
    # Replacing the rows a query must not see by huge values leaves it unchanged.
    rng = _rng(7)
    Kq, Hq, Hk, D = 5, 2, 1, 8
    n_last = 11
    k = rng.standard_normal((n_last, Hk, D))
    v = rng.standard_normal((n_last, Hk, D))
    q = rng.standard_normal((1, Kq, Hq, D))
    o = oracle.decode_attention(q, [k], [v], [n_last], 0.3, Hk)
    for j in range(Kq):
        n = n_last - (Kq - 1 - j)
        k2, v2 = k.copy(), v.copy()
        k2[n:] = 1e3
        v2[n:] = 1e6
        o2 = oracle.decode_attention(q, [k2], [v2], [n_last], 0.3, Hk)
        np.testing.assert_array_equal(o2[0, j], o[0, j])
        if n < n_last:
            assert not np.allclose(o2[0, Kq - 1], o[0, Kq - 1])


def test_rejects_query_with_no_visible_key():
    with pytest.raises(ValueError):
        oracle.decode_attention(np.zeros((1, 3, 1, 4)), [np.zeros((2, 1, 4))], [np.zeros((2, 1, 4))],
                                [2], 1.0, 1)
