"""Oracle: codebook logit projection (float64).

Test infrastructure only (see the package docstring).

TontaubeV1 (audio head paragraph) replaces the language-model head with a
per-stage audio head that projects the transformer state onto that stage's
codebook (16,384 semantic entries or 4,096 acoustic entries, codec
paragraph).  The workloads here use a single bias-free linear map per stage:

  logits[r, v] = sum_k h[r, k] * W[g(r)][v, k]

with g(r) = head_id[r] (the stage of row r's stream), W[g] row-major [V, d].

The audio head TontaubeV1 actually describes (audio head paragraph) has two
layers: it widens the state to 4,096, applies Mish, and projects to the
stage's vocabulary.  ``codebook_head_mlp`` computes that head:

  z[r, f]      = sum_k h[r, k] * W1[g(r)][f, k]            (W1[g] [F, d])
  a[r, f]      = bf16( Mish(z[r, f]) ),  Mish(x) = x * tanh(softplus(x))
  logits[r, v] = sum_f a[r, f] * W2[g(r)][v, f]            (W2[g] [V, F])

Readings where the page leaves a step open: no biases (as for the one-layer
head); Mish as Misra (2019) defines it; the widened activation is stored in
the step's element type (bf16) between the two products, rounded once from
the exact (float64) value to the nearest bfloat16, ties to even (fp32
workloads keep it in float64).
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


def mish(x):
    """x * tanh(softplus(x)) in float64; softplus(x) = log(1 + e^x) evaluated
    as logaddexp(0, x) so that it neither overflows nor loses small values."""
    x = np.asarray(x, np.float64)
    return x * np.tanh(np.logaddexp(0.0, x))


def round_to_bf16_f64(x):
    """Round float64 values to the nearest bfloat16 value (ties to the even
    significand) in one step, returned as float64.  bfloat16 keeps 8
    significant bits and float32's exponent range: a normal value
    x = m * 2^e (0.5 <= |m| < 1) is a multiple of 2^(e-8) after rounding, and
    below the smallest normal 2^-126 the step is the subnormal one, 2^-133.
    Values past the largest finite bfloat16 become infinite."""
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e.astype(np.int64) - 8, -133)
    step = np.ldexp(1.0, q)
    r = np.rint(x / step) * step            # np.rint rounds halves to even
    big = np.abs(r) >= 2.0 ** 128           # past (2 - 2^-7) * 2^127
    return np.where(big, np.copysign(np.inf, x), r)


def codebook_head_mlp(h, W1, W2, head_id=None, act_bf16=True):
    """h [M, d]; W1 [G, F, d]; W2 [G, V, F]; head_id [M] (None = all zero).
    Returns (act [M, F] float64 after Mish and, with act_bf16, bf16 rounding;
    logits [M, V] float64)."""
    W1 = np.asarray(W1)
    W2 = np.asarray(W2)
    if W1.ndim == 2:
        W1, W2 = W1[None], W2[None]
    z = codebook_head(h, W1, head_id)
    a = mish(z)
    if act_bf16:
        a = round_to_bf16_f64(a)
    return a, codebook_head(a, W2, head_id)
