"""GPU statistics: the speculative-sampling theorem and the sampler's
distribution, checked on one large call each (Optimizing Streaming
Text-to-Speech Models ..., "Speculative Decoding for Acoustic Tokens": the
tokens kept by verification follow the target model's distribution, and a
draft is accepted with probability sum_x min(p(x), q(x))).

Every stream sees the same small-vocabulary target and draft rows, its own
drafted tokens (drawn from the draft rows) and uniforms, all seeded.  The
number of tokens a stream emits follows from the per-position acceptance
rates (independent positions), which also fixes how often the bonus token
appears.  The
counts are compared with the target probabilities (float64 softmax) by a
chi-square statistic at a 1e-6 tail, so a kernel that drew from the wrong
distribution (the draft's, an unnormalised residual, a shifted CDF) fails
while the seeded run is stable.
"""

import numpy as np
import pytest
from scipy import stats

from parity import to_torch

pytestmark = pytest.mark.gpu


def _softmax(x, T):
    z = np.asarray(x, np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


def _chi2_ok(counts, probs, what):
    n = counts.sum()
    exp = probs * n
    keep = exp > 0
    assert counts[~keep].sum() == 0, f"{what}: tokens of zero probability drawn"
    chi2 = float((((counts - exp) ** 2)[keep] / exp[keep]).sum())
    crit = float(stats.chi2.isf(1e-6, int(keep.sum()) - 1))
    print(f"{what}: n {n}, chi2 {chi2:.2f} (1e-6 tail {crit:.2f})")
    assert chi2 < crit, (what, chi2, crit, counts.tolist(), (probs * n).round(1).tolist())


@pytest.mark.parametrize("bonus", [False, True])
def test_spec_verify_keeps_the_target_distribution(clm_gpu, bonus):
    rng = np.random.default_rng(2024 + bonus)
    B, K, V, T = 200_000, 3, 6, 1.0
    tl_rows = rng.standard_normal((K + 1, V)).astype(np.float32) * 1.5
    q_rows = np.stack([_softmax(rng.standard_normal(V) * 1.5, 1.0) for _ in range(K)])
    p_rows = np.stack([_softmax(tl_rows[i], T) for i in range(K + 1)])
    tl = np.broadcast_to(tl_rows[None, :K + (1 if bonus else 0)], (B, K + (1 if bonus else 0), V)).copy()
    q = np.broadcast_to(q_rows[None].astype(np.float32), (B, K, V)).copy()
    cum = np.cumsum(q_rows, axis=1)
    drafts = np.stack([np.minimum(np.searchsorted(cum[i], rng.random(B)), V - 1) for i in range(K)], axis=1)
    drafts = drafts.astype(np.int32)
    ua = rng.random((B, K), dtype=np.float32)
    ur = rng.random(B, dtype=np.float32)
    f = clm_gpu.spec_verify_bonus if bonus else clm_gpu.spec_verify
    toks, num = f(to_torch(tl), to_torch(q), to_torch(drafts), to_torch(ua), to_torch(ur), T)
    toks, num = toks.cpu().numpy(), num.cpu().numpy()

    # the first token of every stream follows p_0
    _chi2_ok(np.bincount(toks[:, 0], minlength=V), p_rows[0], f"first token (bonus={bonus})")
    # draft 0 is accepted with probability sum min(p_0, q_0) (kept drafts: num >= 2)
    accepted0 = num >= 2
    alpha = float(np.minimum(p_rows[0], q_rows[0]).sum())
    rate = accepted0.mean()
    sd = np.sqrt(alpha * (1 - alpha) / B)
    print(f"acceptance of draft 0: {rate:.4f} against {alpha:.4f} (sd {sd:.4f})")
    assert abs(rate - alpha) < 5 * sd + 1e-9
    # given draft 0 kept, the second token follows p_1
    sel = num >= 2
    _chi2_ok(np.bincount(toks[sel, 1], minlength=V), p_rows[1], f"second token (bonus={bonus})")
    # drafts and uniforms are independent across positions, so the stream's
    # first rejection is at j with probability alpha_0 ... alpha_{j-1} (1 - alpha_j)
    # and it emits j + 1 tokens; with no rejection it emits K (K + 1 with the bonus)
    alphas = np.minimum(p_rows[:K], q_rows).sum(axis=1)
    for j in range(K + 1):
        pj = float(np.prod(alphas[:j]) * (1.0 - alphas[j] if j < K else 1.0))
        n_j = K + (1 if bonus else 0) if j == K else j + 1
        if not bonus and j >= K - 1:       # a rejection at the last draft and no rejection both emit K
            if j == K:
                continue
            pj += float(np.prod(alphas))
        rate = float((num == n_j).mean())
        sd = np.sqrt(pj * (1 - pj) / B)
        print(f"emitted {n_j}: {rate:.4f} against {pj:.4f} (sd {sd:.4f})")
        assert abs(rate - pj) < 5 * sd + 1e-9, (n_j, rate, pj)
    if bonus:
        # after K accepted drafts the bonus token follows p_K
        allk = num == K + 1
        assert allk.sum() > 1000
        _chi2_ok(np.bincount(toks[allk, K], minlength=V), p_rows[K], "bonus token")
    else:
        assert num.max() <= K


def test_sampler_follows_the_softmax(clm_gpu):
    rng = np.random.default_rng(77)
    M, V, T = 200_000, 7, 0.7
    row = rng.standard_normal(V).astype(np.float32) * 1.2
    logits = np.broadcast_to(row[None], (M, V)).copy()
    u = rng.random(M, dtype=np.float32)
    tok = clm_gpu.sample_or_argmax(to_torch(logits), to_torch(np.full(M, T, np.float32)), to_torch(u)).cpu().numpy()
    _chi2_ok(np.bincount(tok, minlength=V), _softmax(row, T), "sampled tokens")
    # inverse CDF: the token is a non-decreasing function of the uniform
    order = np.argsort(u, kind="stable")
    assert np.all(np.diff(tok[order]) >= 0)
