"""Oracle: codebook logit projection (float64).

Test infrastructure only (see the package docstring).

TontaubeV1 (audio head paragraph) replaces the language-model head with a
per-stage audio head that projects the transformer state onto that stage's
codebook (16,384 semantic entries or 4,096 acoustic entries, codec
paragraph).  The workloads here use a single bias-free linear map per stage:

  logits[r, v] = sum_k h[r, k] * W[g(r)][v, k]

with g(r) = head_id[r] (the stage of row r's stream), W[g] row-major [V, d].
"""

from __future__ import annotations

import numpy as np


def codebook_head(h, W, head_id=None, rows=None):
    """h [M, d]; W [G, V, d]; head_id [M] (None = all zero).  Returns
    logits [M, V] float64 (rows outside ``rows`` stay zero when given)."""
    h = np.asarray(h, np.float64)
    W = np.asarray(W)
    if W.ndim == 2:
        W = W[None]
    G, V, d = W.shape
    M = h.shape[0]
    if h.shape[1] != d:
        raise ValueError("h has width %d, W has %d" % (h.shape[1], d))
    hid = np.zeros(M, np.int64) if head_id is None else np.asarray(head_id, np.int64)
    out = np.zeros((M, V), np.float64)
    Wf = {}
    for r in (range(M) if rows is None else rows):
        g = int(hid[r])
        if not 0 <= g < G:
            raise ValueError("head_id %d out of range" % g)
        if g not in Wf:
            Wf[g] = np.asarray(W[g], np.float64)
        out[r] = Wf[g] @ h[r]
    return out
