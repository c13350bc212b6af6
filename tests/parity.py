"""Parity rules between the GPU library and the oracle, and torch plumbing.

Tolerances (written here, used by every GPU parity test):
  attention outputs and logits: |gpu - ref| <= 2e-2 + 2e-2*|ref| elementwise
  KV append: bit-exact
  argmax tokens: equal, unless the reference's top-2 logit gap is < 1e-3; an
    exempt row must still pick a token whose reference logit is within 1e-3
    of the maximum
  sampled tokens: equal, unless u lies within 1e-4 of either CDF bound of the
    reference token; an exempt row's token must have a reference CDF interval
    that meets [u - 1e-4, u + 1e-4]
  accept/reject: every decision equal, unless |u - p[x]/q| < 1e-4 (then that
    stream's later outputs are exempt); a residual draw follows the sampling
    rule on the reference residual CDF
"""

from __future__ import annotations

import numpy as np

import oracle

ATOL = 2e-2
RTOL = 2e-2
GAP = 1e-3
UEPS = 1e-4


def to_torch(a, device="cuda", bf16=False):
    import torch
    if bf16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def bf16_tensor_to_f32(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def check_close(gpu, ref, what, atol=ATOL, rtol=RTOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu {gpu[i]!r} ref {ref[i]!r}")
    return float(err.max()) if err.size else 0.0


def tolerance_used(gpu, ref, atol=ATOL, rtol=RTOL):
    """The largest |gpu - ref| / (atol + rtol |ref|): 1.0 is the edge of the bar."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    r = np.abs(gpu - ref) / (atol + rtol * np.abs(ref))
    return float(r.max()) if r.size else 0.0


def check_argmax(gpu_tok, ref_logits, what, vocab_valid=None):
    """Returns the number of exempt rows."""
    exempt = 0
    for r, g in enumerate(np.asarray(gpu_tok)):
        row = np.asarray(ref_logits[r], np.float64)
        n = len(row) if vocab_valid is None else int(vocab_valid[r])
        row = row[:n]
        ref_tok = oracle.argmax_token(row.astype(np.float32))
        if g == ref_tok:
            continue
        top2 = np.sort(row)[-2:] if n > 1 else np.array([row[0], -np.inf])
        gap = top2[1] - top2[0]
        assert 0 <= g < n, f"{what} row {r}: token {g} outside [0,{n})"
        assert gap < GAP, f"{what} row {r}: gpu {g} != ref {ref_tok} (gap {gap:.3g})"
        assert row[g] >= row.max() - GAP, f"{what} row {r}: exempt row picked a far token"
        exempt += 1
    return exempt


def _cdf_bounds(weights):
    w = np.asarray(weights, np.float32)
    c = np.cumsum(w, dtype=np.float32)
    C = (c / c[-1]).astype(np.float64)
    lo = np.concatenate([[0.0], C[:-1]])
    return lo, C


def check_sampled(gpu_tok, ref_logits, temperature, uniforms, what, vocab_valid=None):
    exempt = 0
    for r, g in enumerate(np.asarray(gpu_tok)):
        x = np.asarray(ref_logits[r], np.float32)
        n = len(x) if vocab_valid is None else int(vocab_valid[r])
        x = x[:n]
        T = np.float32(temperature[r])
        u = float(uniforms[r])
        ref_tok = oracle.sample_token(x, T, uniforms[r])
        if g == ref_tok:
            continue
        z = x / T
        e = np.exp(z - z.max()).astype(np.float32)
        lo, hi = _cdf_bounds(e)
        near = abs(u - lo[ref_tok]) < UEPS or abs(u - hi[ref_tok]) < UEPS
        assert 0 <= g < n, f"{what} row {r}: token {g} outside [0,{n})"
        assert near, f"{what} row {r}: gpu {g} != ref {ref_tok}, u={u} interval [{lo[ref_tok]}, {hi[ref_tok]})"
        assert lo[g] <= u + UEPS and hi[g] >= u - UEPS, f"{what} row {r}: exempt token {g} far from u"
        exempt += 1
    return exempt


def check_verify(gpu_toks, gpu_num, ref_logits, draft_probs, draft_tokens, u_acc, u_res, T, what,
                 bonus=False):
    """Walks each stream's decisions against the oracle's.  Returns the
    number of exempt streams.  With bonus, ref_logits has K+1 rows and a
    stream whose K drafts are all accepted emits one more token."""
    B, K = draft_tokens.shape
    exempt = 0
    for b in range(B):
        ref = oracle.spec_verify_stream(ref_logits[b], draft_probs[b], draft_tokens[b], u_acc[b], u_res[b], T,
                                        bonus=bonus)
        got = list(np.asarray(gpu_toks[b][:int(gpu_num[b])]))
        assert 1 <= int(gpu_num[b]) <= K + (1 if bonus else 0), f"{what} stream {b}: num_emitted {gpu_num[b]}"
        assert np.all(np.asarray(gpu_toks[b][int(gpu_num[b]):]) == -1), f"{what} stream {b}: padding"
        if got == ref:
            continue
        # find the first difference and decide whether it is exempt
        stream_exempt = False
        for i in range(K):
            p = oracle.target_probs(ref_logits[b][i], T)
            x = int(draft_tokens[b][i])
            qx = np.float32(draft_probs[b][i][x])
            ratio = float(p[x] / qx) if qx > 0 else 0.0
            if qx > 0 and abs(float(u_acc[b][i]) - ratio) < UEPS:
                stream_exempt = True
                break
            ref_accept = qx > 0 and np.float32(u_acc[b][i]) < np.float32(p[x] / qx)
            if ref_accept:
                assert i < len(got) and got[i] == x, f"{what} stream {b} pos {i}: gpu rejected an accept"
                continue
            # reference rejected at i: GPU must emit a residual token at i and stop
            assert len(got) == i + 1, f"{what} stream {b}: gpu accepted at {i} where ref rejected"
            resid = np.maximum(p - np.asarray(draft_probs[b][i], np.float32), np.float32(0))
            if not np.any(resid > 0):
                resid = p
            lo, hi = _cdf_bounds(resid)
            u = float(u_res[b])
            g = got[i]
            rt = ref[i]
            near = abs(u - lo[rt]) < UEPS or abs(u - hi[rt]) < UEPS
            assert near, f"{what} stream {b} pos {i}: residual gpu {g} != ref {rt}"
            assert lo[g] <= u + UEPS and hi[g] >= u - UEPS
            stream_exempt = True
            break
        else:
            if bonus:
                # every draft accepted in the reference: the bonus draw differs
                assert len(got) == K + 1, f"{what} stream {b}: no bonus token after K accepts"
                lo, hi = _cdf_bounds(oracle.target_probs(ref_logits[b][K], T))
                u = float(u_res[b])
                g, rt = got[K], ref[K]
                assert abs(u - lo[rt]) < UEPS or abs(u - hi[rt]) < UEPS, \
                    f"{what} stream {b}: bonus gpu {g} != ref {rt}"
                assert lo[g] <= u + UEPS and hi[g] >= u - UEPS
                stream_exempt = True
        assert stream_exempt, f"{what} stream {b}: {got} vs {ref}"
        exempt += 1
    return exempt
