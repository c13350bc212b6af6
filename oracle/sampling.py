"""Oracle: greedy argmax and temperature sampling of one token per row (float32).

Test infrastructure only (see the package docstring).

* Greedy (temperature 0): TontaubeV1 decodes its later stages at temperature
  zero; the token is the index of the largest logit, the lowest such index
  on ties (the pages fix no tie rule).
* Temperature T > 0: p = softmax(logits / T) (the verification listing of
  "Speculative Decoding for Acoustic Tokens" divides logits by the
  temperature before the softmax).  The draw uses a supplied uniform u in
  [0, 1) by inverse CDF in ascending token order:
      token = min{ i : u < C_i },   C_i = sum_{j<=i} e_j / sum_j e_j
  If rounding leaves u >= every C_i, the last index with e_i > 0 is taken.
* Masking: TontaubeV1 Section 3.3 masks logits outside the stage's target
  vocabulary at sampling time; with ``vocab_valid`` given, indices >= it get
  probability zero and cannot win the argmax.
All arithmetic is float32 (the kernels decide in float32); sums run
sequentially in index order.
"""

from __future__ import annotations

import numpy as np


def argmax_token(logits_row, vocab_valid=None):
    x = np.asarray(logits_row, np.float32)
    n = x.shape[0] if vocab_valid is None else int(vocab_valid)
    if n < 1:
        raise ValueError("empty vocabulary")
    best = 0
    for i in range(1, n):
        if x[i] > x[best]:
            best = i
    return best


def inverse_cdf(weights, u):
    """min{i : u < C_i} for C_i = cumsum(weights)_i / sum(weights), float32."""
    w = np.asarray(weights, np.float32)
    c = np.cumsum(w, dtype=np.float32)          # sequential float32 prefix sums
    total = c[-1]
    C = c / total
    hit = np.nonzero(np.float32(u) < C)[0]
    if hit.size:
        return int(hit[0])
    return int(np.nonzero(w > 0)[0][-1])


def sample_token(logits_row, temperature, u, vocab_valid=None):
    x = np.asarray(logits_row, np.float32)
    n = x.shape[0] if vocab_valid is None else int(vocab_valid)
    z = x[:n] / np.float32(temperature)
    e = np.exp(z - z.max()).astype(np.float32)
    return inverse_cdf(e, u)


def sample_or_argmax(logits, temperature=None, uniforms=None, vocab_valid=None):
    """Row-wise: temperature[r] == 0 (or temperature None) -> argmax, else sample
    with uniforms[r].  Returns int32 [M]."""
    logits = np.asarray(logits, np.float32)
    M = logits.shape[0]
    out = np.empty(M, np.int32)
    for r in range(M):
        vv = None if vocab_valid is None else int(vocab_valid[r])
        T = 0.0 if temperature is None else float(temperature[r])
        if T == 0.0:
            out[r] = argmax_token(logits[r], vv)
        else:
            out[r] = sample_token(logits[r], T, uniforms[r], vv)
    return out
