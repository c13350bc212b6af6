"""Oracle: speculative verification of K drafted speech tokens per stream (float32).

Test infrastructure only (see the package docstring).

The rule ("Speculative Decoding for Acoustic Tokens", Optimizing Streaming
Text-to-Speech Models for Sub-50 Millisecond Latency): one target pass gives
a distribution p_i for each of the K drafted positions (the target logits
over the temperature, softmaxed; at T = 0 the one-hot argmax).  Draft i,
token x_i with draft probability q_i = draft_probs[i][x_i], is accepted when
q_i > 0 and the supplied uniform u_i is below p_i[x_i] / q_i.  The stream
keeps the drafts before the first rejected position j, and at j emits one
draw from max(p_j - draft_probs[j], 0) normalised; with no rejection every
draft is kept.  Stated that way, the oracle computes all K acceptance
tests at once, finds j as the first failed test, and makes the one draw.

Bonus-token variant (``bonus=True``): the target pass also scores the
position after the last draft, so K+1 target distributions are given; when
no draft is rejected, one more token is drawn from the (K+1)-th target
distribution with u_resample (only one of the residual and bonus draws can
happen).  The blog's 0.28 forward passes per token (section 'Latency
Benchmark Analysis') matches this variant at its alpha = 0.82, K = 4.

Readings where the pages leave a step open: no bonus token after K accepts
in the default form; the random numbers are supplied (u_accept [B,K],
u_resample [B]) and every draw is by inverse CDF in ascending token order;
if the residual has zero mass (only possible when p equals the draft
distribution) the draw is from p; streams are independent.  Outputs: the
emitted tokens padded with -1 to length K, and their count (1..K).
"""

from __future__ import annotations

import numpy as np

from .sampling import argmax_token, inverse_cdf


def target_probs(logits_row, temperature):
    x = np.asarray(logits_row, np.float32)
    if temperature == 0.0:
        p = np.zeros_like(x)
        p[argmax_token(x)] = 1.0
        return p
    z = x / np.float32(temperature)
    e = np.exp(z - z.max()).astype(np.float32)
    total = np.cumsum(e, dtype=np.float32)[-1]
    return e / total


def spec_verify_stream(target_logits, draft_probs, draft_tokens, u_accept, u_resample, temperature,
                       bonus=False):
    K = len(draft_tokens)
    if target_logits.shape[0] != K + (1 if bonus else 0):
        raise ValueError("target rows must be K (K + 1 with a bonus token)")
    x = np.asarray(draft_tokens, np.int64)
    qrows = np.asarray(draft_probs, np.float32)
    p = np.stack([target_probs(target_logits[i], temperature) for i in range(K)])   # [K, V]
    q_x = qrows[np.arange(K), x]
    p_x = p[np.arange(K), x]
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(q_x > 0, p_x / np.where(q_x > 0, q_x, np.float32(1)), np.float32(0)).astype(np.float32)
    accepted = (q_x > 0) & (np.asarray(u_accept, np.float32) < ratio)
    rejected = np.nonzero(~accepted)[0]
    if rejected.size:
        j = int(rejected[0])
        resid = np.maximum(p[j] - qrows[j], np.float32(0)).astype(np.float32)
        if not np.any(resid > 0):
            resid = p[j]
        return [int(t) for t in x[:j]] + [inverse_cdf(resid, u_resample)]
    out = [int(t) for t in x]
    if bonus:
        out.append(inverse_cdf(target_probs(target_logits[K], temperature), u_resample))
    return out


def spec_verify(target_logits, draft_probs, draft_tokens, u_accept, u_resample, temperature,
                streams=None, bonus=False):
    """Batched form: target_logits [B,K,V] ([B,K+1,V] with bonus), draft_probs
    [B,K,V]; returns (out_tokens [B,K] ([B,K+1] with bonus) int32 padded with
    -1, num_emitted [B] int32)."""
    B, K = draft_tokens.shape
    out = np.full((B, K + (1 if bonus else 0)), -1, np.int32)
    num = np.zeros(B, np.int32)
    for b in (range(B) if streams is None else streams):
        toks = spec_verify_stream(target_logits[b], draft_probs[b], draft_tokens[b],
                                  u_accept[b], u_resample[b], temperature, bonus=bonus)
        out[b, :len(toks)] = toks
        num[b] = len(toks)
    return out, num
