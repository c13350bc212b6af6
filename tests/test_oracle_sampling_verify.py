"""Pins for the sampler and speculative-verification oracles (CPU only).

Closed forms, brute force on tiny vocabularies, the speculative-sampling
theorem (emitted tokens follow the target distribution; acceptance rate
sum_x min(p, q)), the acceptance figure the speculative-decoding blog
prints (tests/golden/spec_acceptance_blog.json), and, for the bonus-token
variant, the blog's passes-per-token figure
(tests/golden/spec_passes_per_token_blog.json).
"""

import json
import math
import os

import numpy as np
import pytest
from scipy import stats

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- argmax -----
def test_argmax_brute_force_with_planted_ties():
    rng = np.random.default_rng(20)
    for trial in range(300):
        V = int(rng.integers(1, 17))
        x = rng.integers(-3, 4, size=V).astype(np.float32)   # many ties
        brute = min(range(V), key=lambda i: (-float(x[i]), i))  # largest value, then lowest index
        assert oracle.argmax_token(x) == brute
        vv = int(rng.integers(1, V + 1))
        brute_m = min(range(vv), key=lambda i: (-float(x[i]), i))
        assert oracle.argmax_token(x, vv) == brute_m


# ---------------------------------------------------------------- sampling ---
def test_equal_logits_sample_floor_u_times_V():
    V = 10
    logits = np.full(V, 0.37, np.float32)
    for k in range(V):
        u = np.float32((k + 0.5) / V)
        assert oracle.sample_token(logits, 0.7, u) == k


def test_two_token_threshold_closed_form():
    l0, l1, T = 0.4, 1.1, 0.7
    thr = 1.0 / (1.0 + math.exp((l1 - l0) / T))       # P(token 0)
    x = np.array([l0, l1], np.float32)
    assert oracle.sample_token(x, T, np.float32(thr - 1e-4)) == 0
    assert oracle.sample_token(x, T, np.float32(thr + 1e-4)) == 1


def test_peaked_and_zero_u_and_mask():
    x = np.zeros(7, np.float32)
    x[4] = 200.0
    for u in np.linspace(0, 0.999, 17, dtype=np.float32):
        assert oracle.sample_token(x, 0.7, u) == 4
    y = np.array([-1e30, -1e30, 0.0, 0.5], np.float32)   # exp underflows to 0 for the first two
    assert oracle.sample_token(y, 1.0, np.float32(0.0)) == 2
    z = np.array([0.0, 0.1, 9.0, 9.5], np.float32)
    for u in np.linspace(0, 0.999, 11, dtype=np.float32):
        assert oracle.sample_token(z, 1.0, u, vocab_valid=2) in (0, 1)
    assert oracle.argmax_token(z, 2) == 1


def test_sampling_histogram_matches_softmax():
    rng = np.random.default_rng(21)
    V, T, n = 6, 0.7, 60000
    x = rng.standard_normal(V).astype(np.float32)
    u = rng.random(n, dtype=np.float32)
    toks = np.array([oracle.sample_token(x, T, ui) for ui in u])
    p = np.exp(x.astype(np.float64) / T)
    p /= p.sum()
    counts = np.bincount(toks, minlength=V)
    chi = stats.chisquare(counts, p * n)
    assert chi.pvalue > 1e-4, chi


def test_sample_or_argmax_rowwise_dispatch():
    x = np.array([[0.1, 0.9, 0.3], [2.0, 0.0, 0.0]], np.float32)
    toks = oracle.sample_or_argmax(x, temperature=np.array([0.0, 1.0], np.float32),
                                   uniforms=np.array([0.5, 0.0], np.float32))
    assert toks.tolist() == [1, 0]


# ---------------------------------------------------------------- verify -----
def _probs(rng, V):
    p = rng.random(V) + 0.05
    return (p / p.sum()).astype(np.float32)


def test_identical_draft_and_target_accept_everything():
    rng = np.random.default_rng(30)
    K, V, T = 5, 9, 0.7
    logits = rng.standard_normal((K, V)).astype(np.float32)
    q = np.stack([oracle.target_probs(logits[i], T) for i in range(K)])
    for trial in range(50):
        drafts = rng.integers(0, V, size=K)
        u = rng.random(K, dtype=np.float32) * np.float32(0.9999)
        out = oracle.spec_verify_stream(logits, q, drafts, u, np.float32(0.5), T)
        assert out == list(drafts)


def test_zero_target_or_zero_draft_probability_rejects():
    V, T = 4, 1.0
    logits = np.array([[0.0, -1e30, 0.0, 0.0]], np.float32)   # p[1] = 0
    q = np.array([[0.25, 0.25, 0.25, 0.25]], np.float32)
    out = oracle.spec_verify_stream(logits, q, np.array([1]), np.array([0.0], np.float32), np.float32(0.1), T)
    # rejected; residual = max(p - q, 0) = 1/3 - 1/4 on {0, 2, 3}; u=0.1 -> token 0
    assert out == [0]
    q0 = np.array([[0.0, 0.5, 0.5, 0.0]], np.float32)          # q[x] = 0 for x = 0
    out = oracle.spec_verify_stream(np.zeros((1, V), np.float32), q0, np.array([0]),
                                    np.array([0.0], np.float32), np.float32(0.9), T)
    assert len(out) == 1 and out[0] in (0, 3)                   # residual lives where p > q


def test_greedy_verification_at_zero_temperature():
    rng = np.random.default_rng(31)
    K, V = 6, 11
    for trial in range(100):
        logits = rng.standard_normal((K, V)).astype(np.float32)
        amax = [oracle.argmax_token(l) for l in logits]
        drafts = np.array([a if rng.random() < 0.7 else (a + 1) % V for a in amax])
        q = np.stack([_probs(rng, V) for _ in range(K)])
        out = oracle.spec_verify_stream(logits, q, drafts, rng.random(K, dtype=np.float32),
                                        rng.random(dtype=np.float32), 0.0)
        j = 0
        while j < K and drafts[j] == amax[j]:
            j += 1
        expect = list(drafts[:j]) + ([amax[j]] if j < K else [])
        assert out == expect


def _run_trials(p_logits, q, T, n, rng, bonus=False):
    """Draw drafts from q and run n verifications; returns emitted lists."""
    K, V = q.shape
    cdf = np.cumsum(q.astype(np.float64), axis=1)
    outs = []
    for _ in range(n):
        drafts = np.array([min(int(np.searchsorted(cdf[i], rng.random(), side="right")), V - 1)
                           for i in range(K)])
        outs.append(oracle.spec_verify_stream(p_logits, q, drafts, rng.random(K, dtype=np.float32),
                                              rng.random(dtype=np.float32), T, bonus=bonus))
    return outs


@pytest.mark.parametrize("V,K", [(2, 1), (3, 2), (5, 3), (8, 2)])
def test_emitted_tokens_follow_the_target_distribution(V, K):
    rng = np.random.default_rng(40 + V)
    T = 0.7
    logits = rng.standard_normal((K, V)).astype(np.float32) * 1.5
    q = np.stack([_probs(rng, V) for _ in range(K)])
    p = [oracle.target_probs(logits[i], T).astype(np.float64) for i in range(K)]
    n = 20000
    outs = _run_trials(logits, q, T, n, rng)
    first = np.bincount([o[0] for o in outs], minlength=V)
    assert stats.chisquare(first, p[0] / p[0].sum() * n).pvalue > 1e-4
    # acceptance rate at position 0 is sum_x min(p(x), q(x)); with K >= 2 an
    # accept at position 0 shows as a second emitted token
    if K > 1:
        acc = sum(1 for o in outs if len(o) > 1)
        alpha = float(np.minimum(p[0], q[0]).sum())
        assert stats.binomtest(acc, n, alpha).pvalue > 1e-4
        second = [o[1] for o in outs if len(o) > 1]
        cnt = np.bincount(second, minlength=V)
        assert stats.chisquare(cnt, p[1] / p[1].sum() * len(second)).pvalue > 1e-4


def test_first_token_distribution_on_a_uniform_grid():
    # V = 3, K = 2: average over the draft token (weighted by q) and a fine
    # midpoint grid of (u_accept, u_resample); the first emitted token must
    # have probability p0 up to the grid resolution.
    rng = np.random.default_rng(50)
    V, K, T, N = 3, 2, 0.7, 400
    logits = rng.standard_normal((K, V)).astype(np.float32)
    q = np.stack([_probs(rng, V) for _ in range(K)])
    p0 = oracle.target_probs(logits[0], T).astype(np.float64)
    grid = ((np.arange(N) + 0.5) / N).astype(np.float32)
    prob = np.zeros(V)
    for x in range(V):
        counts = np.zeros(V)
        for ua in grid:
            for ur in grid[::8]:
                out = oracle.spec_verify_stream(logits, q, np.array([x, 0]), np.array([ua, 0.5], np.float32), ur, T)
                counts[out[0]] += 1
        prob += q[0, x] * counts / counts.sum()
    np.testing.assert_allclose(prob, p0, atol=8e-3)


def test_acceptance_figure_from_the_blog():
    g = json.load(open(os.path.join(GOLDEN, "spec_acceptance_blog.json")))
    alpha, K = g["alpha"], g["K"]
    # target p = [1, 0] (logit gap drives the second probability to 0), draft
    # q = [alpha, 1 - alpha]: sum min(p, q) = alpha at every position.
    logits = np.tile(np.array([0.0, -1e30], np.float32), (K, 1))
    q = np.tile(np.array([alpha, 1 - alpha], np.float32), (K, 1))
    rng = np.random.default_rng(60)
    outs = _run_trials(logits, q, 0.7, 20000, rng)
    mean_emitted = np.mean([len(o) for o in outs])
    closed = (1 - alpha ** K) / (1 - alpha)
    assert abs(mean_emitted - closed) < 0.03
    assert abs(closed - g["reported_speedup"]) < g["tolerance"]
    assert abs((1 - alpha ** (K + 1)) / (1 - alpha) - g["reported_speedup"]) > g["tolerance"]


def test_bonus_variant_matches_the_blogs_passes_per_token():
    g = json.load(open(os.path.join(GOLDEN, "spec_passes_per_token_blog.json")))
    alpha, K = g["alpha"], g["K"]
    # acceptance probability exactly alpha at every position (target [1, 0],
    # draft [alpha, 1 - alpha]); the bonus row's target is also [1, 0]
    logits = np.tile(np.array([0.0, -1e30], np.float32), (K + 1, 1))
    q = np.tile(np.array([alpha, 1 - alpha], np.float32), (K, 1))
    rng = np.random.default_rng(61)
    outs = _run_trials(logits, q, 0.7, 20000, rng, bonus=True)
    mean_emitted = np.mean([len(o) for o in outs])
    closed = (1 - alpha ** (K + 1)) / (1 - alpha)
    assert abs(mean_emitted - closed) < 0.03
    assert all(1 <= len(o) <= K + 1 for o in outs)
    assert abs(1 / closed - g["reported_passes_per_token"]) < g["tolerance"]
    # the variant without a bonus token does not reproduce the figure
    assert abs((1 - alpha) / (1 - alpha ** K) - g["reported_passes_per_token"]) > g["tolerance"]


@pytest.mark.parametrize("V,K", [(3, 1), (5, 2)])
def test_bonus_token_follows_the_last_target_distribution(V, K):
    # drafts equal to the target distribution are always accepted (u < 1), so
    # every run ends with a bonus draw from the (K+1)-th target row
    rng = np.random.default_rng(70 + V)
    T = 0.7
    logits = rng.standard_normal((K + 1, V)).astype(np.float32) * 1.5
    q = np.stack([oracle.target_probs(logits[i], T) for i in range(K)])
    n = 20000
    outs = _run_trials(logits, q, T, n, rng, bonus=True)
    assert all(len(o) == K + 1 for o in outs)
    p_last = oracle.target_probs(logits[K], T).astype(np.float64)
    cnt = np.bincount([o[K] for o in outs], minlength=V)
    assert stats.chisquare(cnt, p_last / p_last.sum() * n).pvalue > 1e-4


def test_bonus_greedy_verification():
    # T = 0: accepted drafts equal each row's argmax; all accepted -> the
    # bonus token is the argmax of the last row; a mismatch stops without one
    rng = np.random.default_rng(80)
    K, V = 3, 6
    logits = rng.standard_normal((K + 1, V)).astype(np.float32)
    amax = [oracle.argmax_token(logits[i]) for i in range(K + 1)]
    q = np.full((K, V), 1.0 / V, np.float32)
    u = np.full(K, 0.5, np.float32)
    out = oracle.spec_verify_stream(logits, q, np.array(amax[:K]), u, 0.3, 0.0, bonus=True)
    assert out == amax
    drafts = np.array(amax[:K])
    drafts[1] = (drafts[1] + 1) % V
    out = oracle.spec_verify_stream(logits, q, drafts, u, 0.3, 0.0, bonus=True)
    assert out == [amax[0], amax[1]]
    with pytest.raises(ValueError):
        oracle.spec_verify_stream(logits[:K], q, drafts, u, 0.3, 0.0, bonus=True)


def test_batched_verify_pads_with_minus_one():
    x = synth.make_inputs(4, B=3)
    s = x.spec_inputs()
    toks, num = oracle.spec_verify(s["target_logits_iso"], s["draft_probs"], s["draft_tokens"],
                                   s["u_accept"], s["u_resample"], 0.7)
    for b in range(3):
        assert 1 <= num[b] <= x.cfg.Kq
        assert np.all(toks[b, num[b]:] == -1)
        assert np.all(toks[b, :num[b]] >= 0)
        assert np.array_equal(toks[b, :num[b] - 1], s["draft_tokens"][b, :num[b] - 1])


def test_configs_match_the_pages_codec_shapes():
    g = json.load(open(os.path.join(GOLDEN, "codec_shapes_tontaube.json")))
    assert g["semantic_codebook"] == 2 ** g["semantic_bits"]
    assert g["acoustic_codebook"] == 2 ** g["acoustic_bits"]
    rate = g["frame_rate_hz"]
    assert rate * (g["semantic_bits"] + 3 * g["acoustic_bits"]) == g["retained_bit_rate"]
    assert rate * (g["semantic_bits"] + 7 * g["acoustic_bits"]) == g["full_stack_bit_rate"]
    vocabs = {c.V for c in synth.CONFIGS.values()}
    assert vocabs == {g["semantic_codebook"], g["acoustic_codebook"]}
    for c in synth.CONFIGS.values():
        assert c.block_size == g["kv_block_tokens"]
        if c.mode == "spec":
            assert c.temperature == g["verify_temperature"]
