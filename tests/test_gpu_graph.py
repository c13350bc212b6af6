"""The decode step captured as one HIP graph: every C-ABI call only enqueues
kernels on the caller's stream (no allocation, host synchronisation or
memset), so a fixed-shape step can be captured and replayed.  Each replay,
with eager work in between that clears the outputs, is checked against the
oracle's chained step, and the replays must agree bit for bit."""

import math
import sys

import numpy as np
import pytest

import oracle
import synth
from parity import bf16_tensor_to_f32, check_argmax, check_close, check_sampled, check_verify, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield


@pytest.mark.parametrize("cfg,B", [(2, None), (4, None), (5, 24)])
def test_step_graph_replays_match_oracle(clm_gpu, cfg, B):
    import torch
    x = synth.make_inputs(cfg, B=B)
    c = x.cfg
    bf = c.dtype == "bf16"
    kp, vp = x.build_pool(include_new=False)
    k_cache, v_cache = to_torch(kp, bf16=bf), to_torch(vp, bf16=bf)
    bt, kv_len, len_before = to_torch(x.block_table), to_torch(x.kv_len), to_torch(x.len_before)
    k_new, v_new, q, W = (to_torch(a, bf16=bf) for a in (x.k_new, x.v_new, x.q, x.W))
    head_id = to_torch(x.head_id) if c.G > 1 else None
    max_kv = int(x.kv_len.max())
    dev = q.device
    ws = torch.zeros(clm_gpu.decode_attention_workspace_size(c.B, c.Kq, c.H_q, c.H_kv, c.D, max_kv) + 256,
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    logits = torch.empty((c.M, c.V), dtype=torch.float32, device=dev)
    tokens = torch.empty(c.M, dtype=torch.int32, device=dev)
    out_tok = torch.empty((c.B, c.Kq), dtype=torch.int32, device=dev)
    num = torch.empty(c.B, dtype=torch.int32, device=dev)
    temp = uni = spec = None
    if c.mode == "sample":
        temp = torch.full((c.M,), c.temperature, dtype=torch.float32, device=dev)
        uni = to_torch(x.uniforms())
    if c.mode == "spec":
        s = x.spec_inputs()
        spec = tuple(to_torch(s[k]) for k in ("draft_probs", "draft_tokens", "u_accept", "u_resample"))

    def step():
        clm_gpu.kv_cache_append(k_new, v_new, k_cache, v_cache, bt, len_before, block_size=c.block_size)
        clm_gpu.decode_attention(q, k_cache, v_cache, bt, kv_len, max_kv, scale=1.0 / math.sqrt(c.D), out=o,
                                 workspace=ws)
        clm_gpu.codebook_head(o.view(c.M, c.d_model), W, head_id, out=logits)
        if spec is not None:
            clm_gpu.spec_verify(logits.view(c.B, c.Kq, c.V), *spec, c.temperature, out_tokens=out_tok,
                                num_emitted=num)
        else:
            clm_gpu.sample_or_argmax(logits, temp, uni, out=tokens)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (o, logits, tokens, out_tok, num)]

    keys = [x.logical_k(b) for b in range(c.B)]
    vals = [x.logical_v(b) for b in range(c.B)]
    s_np = x.spec_inputs() if c.mode == "spec" else None
    temp_np = np.full(c.M, c.temperature, np.float32) if c.mode == "sample" else None
    u_np = x.uniforms() if c.mode == "sample" else None
    ref = oracle.decode_step(x.f32(x.q), keys, vals, x.kv_len, 1.0 / math.sqrt(c.D), c.H_kv, x.f32(x.W),
                             x.head_id, bf, mode=c.mode,
                             temperature=(c.temperature if c.mode == "spec" else temp_np), uniforms=u_np,
                             spec=s_np)

    def check_against_oracle(got, what):
        g_o, g_logits, g_tok, g_out, g_num = got
        check_close(bf16_tensor_to_f32(g_o), ref["o"], f"{what} attention")
        check_close(g_logits.cpu().numpy(), ref["logits"], f"{what} logits")
        if c.mode == "spec":
            check_verify(g_out.cpu().numpy(), g_num.cpu().numpy(), ref["logits"].reshape(c.B, c.Kq, c.V),
                         s_np["draft_probs"], s_np["draft_tokens"], s_np["u_accept"], s_np["u_resample"],
                         c.temperature, f"{what} verify")
        elif c.mode == "sample":
            check_sampled(g_tok.cpu().numpy(), ref["logits"], temp_np, u_np, f"{what} sample")
        else:
            check_argmax(g_tok.cpu().numpy(), ref["logits"], f"{what} argmax")

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    first = None
    for r in range(3):
        for t in (o, logits, tokens, out_tok, num):   # eager work between replays
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        check_against_oracle(got, f"graph c{cfg} replay {r}")
        if first is None:
            first = got
            continue
        for name, a, b in zip(("o", "logits", "tokens", "out_tokens", "num_emitted"), got, first):
            if name in ("tokens",) and c.mode == "spec":
                continue
            if name in ("out_tokens", "num_emitted") and c.mode != "spec":
                continue
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), (cfg, r, name)
    print(f"graph c{cfg}: 3 replays match the oracle and each other bit for bit")
