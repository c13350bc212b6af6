"""Host logic of bench.py that needs no GPU: the parity summary the benchmark
line carries (the timed step's outputs against the oracle's)."""

import types

import numpy as np
import torch

import bench


def _case(seed=0, B=6, V=50):
    rng = np.random.default_rng(seed)
    c = types.SimpleNamespace(Kq=1)
    o_ref = rng.standard_normal((B, 1, 2, 8))
    l_ref = rng.standard_normal((B, V)).astype(np.float32)
    l_ref[:, 7] = l_ref.max(axis=1) + 1.0            # a clear winner per row
    ref = {"o": o_ref, "logits": l_ref}
    o = torch.from_numpy(o_ref.astype(np.float32))
    logits = torch.from_numpy(l_ref.copy())
    tokens = torch.from_numpy(np.argmax(l_ref, axis=1).astype(np.int32))
    return c, ref, o, logits, tokens


def test_parity_summary_passes_on_the_oracle_itself():
    c, ref, o, logits, tokens = _case()
    p = bench.parity_of_step(c, list(range(6)), ref, o, logits, tokens)
    assert p["pass"] and p["tokens_equal"] == 6 and p["tokens_exempt"] == 0
    assert p["attention_bar_share"] < 1e-5 and p["logits_bar_share"] == 0.0


def test_parity_summary_flags_errors_and_exempts_near_ties():
    c, ref, o, logits, tokens = _case(1)
    # a near tie in row 2: the GPU may pick the runner-up
    ref["logits"][2, 9] = ref["logits"][2, 7] - 5e-4
    logits[2, 9] = float(ref["logits"][2, 9])
    tokens[2] = 9
    p = bench.parity_of_step(c, list(range(6)), ref, o, logits, tokens)
    assert p["pass"] and p["tokens_exempt"] == 1 and p["tokens_equal"] == 5
    # a wrong token where the gap is clear fails
    tokens[3] = 0
    assert not bench.parity_of_step(c, list(range(6)), ref, o, logits, tokens)["pass"]
    tokens[3] = 7
    # an attention output outside 2e-2 + 2e-2 |ref| fails
    o[4, 0, 1, 3] += 0.5
    p = bench.parity_of_step(c, list(range(6)), ref, o, logits, tokens)
    assert not p["pass"] and p["attention_bar_share"] > 1.0
