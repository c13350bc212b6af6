"""Oracle: speculative verification of K drafted speech tokens per stream (float32).

Test infrastructure only (see the package docstring).

"Speculative Decoding for Acoustic Tokens" (Optimizing Streaming
Text-to-Speech Models for Sub-50 Millisecond Latency): one target pass gives a
distribution for each of the K drafted positions; the drafts are checked in
order:

  for i = 0 .. K-1:
      p   = softmax(target_logits[i] / T)     (T = 0: one-hot at the argmax)
      x   = draft_tokens[i],  q = draft_probs[i][x]
      accept iff q > 0 and u_accept[i] < p[x] / q
      accept -> emit x and go on
      reject -> emit a draw from max(p - draft_probs[i], 0), normalised,
                and stop
Bonus-token variant (``bonus=True``): the target pass also scores the
position after the last draft, so K+1 target distributions are given; when
all K drafts are accepted, one more token is drawn from the (K+1)-th target
distribution with u_resample (only one of the residual and bonus draws can
happen).  The blog's 0.28 forward passes per token (section 'Latency
Benchmark Analysis') matches this variant at its alpha = 0.82, K = 4.
Readings where the pages leave a step open: no bonus token after K accepts
in the default form;
the random numbers are supplied (u_accept [B,K], u_resample [B]) and the
residual draw is by inverse CDF in ascending token order; if the residual has
zero mass (only possible when p equals the draft distribution) the draw is
from p; streams are independent.  Outputs: the emitted tokens padded with -1
to length K, and their count (1..K).
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
    out = []
    for i in range(K):
        p = target_probs(target_logits[i], temperature)
        qrow = np.asarray(draft_probs[i], np.float32)
        x = int(draft_tokens[i])
        qx = qrow[x]
        accepted = bool(qx > 0) and bool(np.float32(u_accept[i]) < np.float32(p[x] / qx))
        if accepted:
            out.append(x)
            continue
        resid = np.maximum(p - qrow, np.float32(0)).astype(np.float32)
        if not np.any(resid > 0):
            resid = p
        out.append(inverse_cdf(resid, u_resample))
        break
    else:
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
