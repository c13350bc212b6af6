"""The multi-step decode loop captured as one HIP graph (clm_decode_loop_*),
against the oracle run step by step.

Each case runs n_steps steps: every step appends Kq new rows per stream
(rotary at logical positions in one case), attends, projects and picks tokens
(greedy, sampling, or speculative verification), then the lengths advance on
the device - by Kq, or by the number of tokens verification kept.  The oracle
follows the same trajectory from its own decisions: per step the attention
outputs, logits and tokens are compared by the parity rules, and at the end
the lengths and (without rotary) the whole cache bit for bit.  One case runs
its live streams inside a larger captured batch padded with idle streams, as
a set of captured batch sizes would; one runs the loop twice from the same
state and requires identical bits.  A stream whose verification decision was
exempt (a uniform within 1e-4 of its ratio) leaves the comparison from then
on, since its trajectory may legitimately differ.
"""

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


def _pages(n, bs):
    return (np.asarray(n, np.int64) + bs - 1) // bs


def _loop_case(clm_gpu, cfg, B_live, B_cap, n_steps, rope=False, use_ws=True, replay=False, bonus=False,
               mlp=False):
    import torch
    x = synth.make_inputs(cfg, B=B_live)
    c = x.cfg
    bf = c.dtype == "bf16"
    bs, Kq, Hk, Hq, D, V, M_cap = c.block_size, c.Kq, c.H_kv, c.H_q, c.D, c.V, B_cap * c.Kq
    f32 = x.f32
    # ---- pool and block table with room for n_steps * Kq more tokens per
    # stream; idle padding streams get pages of their own
    kp, vp, bt, nb = x.pool_with_room((n_steps - 1) * Kq, idle_streams=B_cap - B_live)
    lb0 = np.concatenate([x.len_before, np.zeros(B_cap - B_live, np.int32)]).astype(np.int32)
    offset = 1000
    pos0 = (lb0[:, None] + offset + np.arange(Kq)[None, :]).astype(np.int32)

    # ---- per-step inputs [n_steps, B_cap, ...] (padding rows zero)
    def padded(a, rows=B_cap):
        out = np.zeros((rows,) + a.shape[1:], a.dtype)
        out[:a.shape[0]] = a
        return out
    steps = [x.step_arrays(s) for s in range(n_steps)]
    k_new = np.stack([padded(k) for k, _, _ in steps])
    v_new = np.stack([padded(v) for _, v, _ in steps])
    q_all = np.stack([padded(q) for _, _, q in steps])
    head_id = np.concatenate([x.head_id, np.zeros(M_cap - c.M, np.int32)]) if c.G > 1 else None
    dev = torch.device("cuda")
    T = lambda a, b16=False: to_torch(np.ascontiguousarray(a), bf16=b16)
    k_cache, v_cache = T(kp, bf), T(vp, bf)
    g = dict(k_cache=k_cache, v_cache=v_cache, block_table=T(bt), len_before=T(lb0), kv_len=T(lb0 + Kq),
             k_new=T(k_new, bf), v_new=T(v_new, bf), q=T(q_all, bf), W=T(x.W, bf),
             head_id=None if head_id is None else T(head_id))
    mlp_w = None
    if mlp:             # TontaubeV1's two-layer head: d -> 4096 -> Mish -> V per stage, N(0, 0.02) weights
        assert c.mode == "greedy" and bf
        wr = np.random.default_rng(4096 + cfg)
        F = 4096
        W1 = synth.f32_to_bf16_bits((wr.standard_normal((c.G, F, c.d_model)) * 0.02).astype(np.float32))
        W2 = synth.f32_to_bf16_bits((wr.standard_normal((c.G, V, F)) * 0.02).astype(np.float32))
        mlp_w = (f32(W1), f32(W2))
        g["W"], g["W2"] = T(W1, True), T(W2, True)
    g["o"] = torch.empty_like(g["q"])
    g["logits"] = torch.empty((n_steps, M_cap, V), dtype=torch.float32, device=dev)
    if rope:
        g["positions"] = T(pos0)
    spec_np = None
    if c.mode == "spec":
        spec_np = [x.spec_inputs(s) for s in range(n_steps)]
        if bonus:           # Kq queries: the last kept token, then Kq - 1 drafts
            for sp in spec_np:
                for k in ("draft_probs", "draft_tokens", "u_accept"):
                    sp[k] = np.ascontiguousarray(sp[k][:, :Kq - 1])
        g["draft_probs"] = T(np.stack([padded(sp["draft_probs"]) for sp in spec_np]))
        g["draft_tokens"] = T(np.stack([padded(sp["draft_tokens"]) for sp in spec_np]))
        g["u_accept"] = T(np.stack([padded(sp["u_accept"]) for sp in spec_np]))
        g["u_resample"] = T(np.stack([padded(sp["u_resample"]) for sp in spec_np]))
        g["out_tokens"] = torch.empty((n_steps, B_cap, Kq), dtype=torch.int32, device=dev)
        g["num_emitted"] = torch.empty((n_steps, B_cap), dtype=torch.int32, device=dev)
    else:
        g["tokens"] = torch.empty((n_steps, M_cap), dtype=torch.int32, device=dev)
    temp_np = uni_np = None
    if c.mode == "sample":
        temp_np = np.full((n_steps, M_cap), c.temperature, np.float32)
        temp_np[:, c.M:] = 0.0
        uni_np = np.stack([padded(x.uniforms_step(s), M_cap) for s in range(n_steps)])
        g["temperature"], g["uniforms"] = T(temp_np), T(uni_np)
    max_kv = int((lb0 + n_steps * Kq).max())
    ws = None
    if use_ws:
        need_ws = clm_gpu.decode_attention_workspace_size(B_cap, Kq, Hq, Hk, D, max_kv)
        ws = torch.empty(need_ws + 256, dtype=torch.uint8, device=dev)
        ws = ws[(-ws.data_ptr()) % 256:]
    initial = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in g.items()}
    loop = clm_gpu.DecodeLoop(max_kv_len=max_kv, mode="spec_bonus" if bonus else c.mode,
                              spec_temperature=c.temperature, attn_workspace=ws, block_size=bs, rope_base=1.0e6, **g)
    loop.launch()
    torch.cuda.synchronize()

    # ---- the oracle, step by step from its own decisions
    scale = 1.0 / math.sqrt(D)
    keys = [x.logical_k(b)[:x.len_before[b]] for b in range(B_live)]
    vals = [x.logical_v(b)[:x.len_before[b]] for b in range(B_live)]
    lb = x.len_before.astype(np.int64).copy()
    live = np.ones(B_live, bool)
    kp_ref, vp_ref = kp.copy(), vp.copy()
    Wf = f32(x.W)
    for s in range(n_steps):
        kn, vn, qs = steps[s]
        kf, vf, qf = f32(kn), f32(vn), f32(qs)
        if rope:
            pos = (lb[:, None] + offset + np.arange(Kq)[None, :])
            qf = oracle.rope(qf, pos[:, :, None], 1.0e6)
            kf = oracle.rope(kf, pos[:, :, None], 1.0e6)
            if bf:          # the cache and the rotated queries hold the step's element type
                qf, kf = oracle.round_to_bf16(qf), oracle.round_to_bf16(kf)
            qf, kf = qf.astype(np.float32), kf.astype(np.float32)
        ks = [np.concatenate([keys[b], kf[b]]) for b in range(B_live)]
        vs = [np.concatenate([vals[b], vf[b]]) for b in range(B_live)]
        kv_len = (lb + Kq).astype(np.int32)
        sp = spec_np[s] if spec_np else None
        if mlp:             # attention as in any step, then the two-layer head and the argmax
            ref = oracle.decode_step(qf, ks, vs, kv_len, scale, Hk, Wf, x.head_id if c.G > 1 else None, bf)
            _, lg = oracle.codebook_head_mlp(ref["h"], mlp_w[0], mlp_w[1], x.head_id if c.G > 1 else None)
            ref["logits"] = lg.astype(np.float32)
            ref["tokens"] = oracle.sample_or_argmax(ref["logits"])
        elif bonus:         # attention and logits as in any step, then the bonus-token verification
            ref = oracle.decode_step(qf, ks, vs, kv_len, scale, Hk, Wf, None, bf)
            ref["out_tokens"], ref["num_emitted"] = oracle.spec_verify(
                ref["logits"].reshape(B_live, Kq, V), sp["draft_probs"], sp["draft_tokens"], sp["u_accept"],
                sp["u_resample"], c.temperature, bonus=True)
        else:
            ref = oracle.decode_step(qf, ks, vs, kv_len, scale, Hk, Wf, x.head_id if c.G > 1 else None, bf,
                                     mode=c.mode,
                                     temperature=(c.temperature if c.mode == "spec" else
                                                  (temp_np[s, :c.M] if temp_np is not None else None)),
                                     uniforms=None if uni_np is None else uni_np[s, :c.M], spec=sp)
        sel = np.nonzero(live)[0]
        rows = (sel[:, None] * Kq + np.arange(Kq)[None, :]).reshape(-1)
        o_g = bf16_tensor_to_f32(g["o"][s])[:B_live]
        lg_g = g["logits"][s].cpu().numpy()[:c.M]
        check_close(o_g[sel], ref["o"][sel], f"loop c{cfg} step {s} attention")
        check_close(lg_g[rows], ref["logits"][rows], f"loop c{cfg} step {s} logits")
        if c.mode == "spec":
            ot = g["out_tokens"][s].cpu().numpy()[:B_live]
            ne = g["num_emitted"][s].cpu().numpy()[:B_live]
            rl = ref["logits"].reshape(B_live, Kq, V)
            check_verify(ot[sel], ne[sel], rl[sel], sp["draft_probs"][sel], sp["draft_tokens"][sel],
                         sp["u_accept"][sel], sp["u_resample"][sel], c.temperature, f"loop c{cfg} step {s} verify",
                         bonus=bonus)
            add = ref["num_emitted"].astype(np.int64)
            for b in sel:
                if ne[b] != add[b] or not np.array_equal(ot[b], ref["out_tokens"][b]):
                    live[b] = False             # exempt decision: trajectories may part here
        else:
            tk = g["tokens"][s].cpu().numpy()[:c.M]
            if c.mode == "sample":
                check_sampled(tk[rows], ref["logits"][rows], temp_np[s, rows], uni_np[s, rows],
                              f"loop c{cfg} step {s} sample")
            else:
                check_argmax(tk[rows], ref["logits"][rows], f"loop c{cfg} step {s} argmax")
            add = np.full(B_live, Kq, np.int64)
        # the oracle's append of this step's rows (plain-append cases), then advance
        if not rope:
            kp_ref, vp_ref = oracle.kv_cache_append(kp_ref, vp_ref, bt[:B_live], lb.astype(np.int32),
                                                    kn, vn, bs)
        for b in range(B_live):
            keys[b] = ks[b][:lb[b] + add[b]]
            vals[b] = vs[b][:lb[b] + add[b]]
        lb = lb + add
    lb_g = g["len_before"].cpu().numpy()
    kvl_g = g["kv_len"].cpu().numpy()
    assert np.array_equal(lb_g[:B_live][live], lb[live]), "lengths after the loop"
    assert np.array_equal(kvl_g[:B_live][live], (lb + Kq)[live])
    idle_adv = (g["num_emitted"].cpu().numpy()[:, B_live:].sum(0) if c.mode == "spec"
                else np.full(B_cap - B_live, n_steps * Kq))
    assert np.array_equal(lb_g[B_live:], idle_adv), "idle streams advance too"
    if rope:
        assert np.array_equal(g["positions"].cpu().numpy()[:B_live][live],
                              (lb[:, None] + offset + np.arange(Kq)[None, :])[live])
    elif live.all():
        dt_ = np.int16 if bf else np.uint32
        kb = k_cache.view(torch.int16).cpu().numpy() if bf else k_cache.cpu().numpy().view(np.uint32)
        vb = v_cache.view(torch.int16).cpu().numpy() if bf else v_cache.cpu().numpy().view(np.uint32)
        live_blocks = np.unique(bt[:B_live])
        np.testing.assert_array_equal(kb[live_blocks], kp_ref.view(dt_)[live_blocks], err_msg="cache keys")
        np.testing.assert_array_equal(vb[live_blocks], vp_ref.view(dt_)[live_blocks], err_msg="cache values")
    if replay:
        first = {k: g[k].clone() for k in ("o", "logits", "tokens", "len_before", "k_cache") if k in g}
        for k, v in initial.items():
            if isinstance(v, torch.Tensor) and k not in ("W",):
                g[k].copy_(v)
        torch.cuda.synchronize()
        loop.launch()
        torch.cuda.synchronize()
        for k, v in first.items():
            a, b_ = g[k], v
            if a.dtype == torch.bfloat16:          # bits, so that NaN in empty slots compares equal
                a, b_ = a.view(torch.int16), b_.view(torch.int16)
            elif a.dtype == torch.float32:
                a, b_ = a.view(torch.int32), b_.view(torch.int32)
            assert torch.equal(a, b_), f"second launch differs in {k}"
    loop.close()
    print(f"loop c{cfg}: {n_steps} steps, {B_live} live of {B_cap}, {int((~live).sum())} streams parted on exempt "
          f"decisions")


def test_loop_greedy_rope_replay(clm_gpu):
    """256-stream mix (24 streams), 4 steps with rotary at logical positions;
    the loop launched twice from the same state gives the same bits."""
    _loop_case(clm_gpu, 5, 24, 24, 4, rope=True, replay=True)


def test_loop_full_size_256_streams(clm_gpu):
    """The graph loop at the size the benchmark times it: all 256 streams of
    the log-uniform 64..8192 mix, 2 steps (1024-token splits, merge pass),
    every stream's attention, logits and token against the oracle, and the
    whole cache bit for bit at the end."""
    _loop_case(clm_gpu, 5, 256, 256, 2)


def test_loop_speculative(clm_gpu):
    """32 streams x 6-query blocks, 4 steps; lengths advance by the tokens kept."""
    _loop_case(clm_gpu, 4, 32, 32, 4)


def test_loop_speculative_rope(clm_gpu):
    """The 6-query blocks with rotary embedding at logical positions, 3 steps:
    the positions advance by the tokens kept, like the lengths, so the next
    block's queries and keys are rotated where its tokens really sit."""
    _loop_case(clm_gpu, 4, 32, 32, 3, rope=True)


def test_loop_speculative_bonus_token(clm_gpu):
    """The same blocks with a bonus token: the 6 queries score the last kept
    token and 5 drafts, and a stream that keeps all 5 drafts emits a sixth
    token from the last target row; 4 steps, lengths advance by 1..6."""
    _loop_case(clm_gpu, 4, 32, 32, 4, bonus=True)


def test_loop_sampling_padded_bucket_static_scratch(clm_gpu):
    """12 live streams in a 16-stream captured batch (4 idle), temperature
    sampling, attention partials in the library's static scratch."""
    sizes = [16, 64, 256]
    assert clm_gpu.pick_bucket(sizes, 12) == 0
    _loop_case(clm_gpu, 2, 12, sizes[clm_gpu.pick_bucket(sizes, 12)], 3, use_ws=False)


def test_loop_two_layer_head(clm_gpu):
    """TontaubeV1's two-layer Mish head in the loop: 64 streams over three
    stage heads, 3 steps, greedy; the activation scratch is reused by every
    step."""
    _loop_case(clm_gpu, 3, 64, 64, 3, mlp=True)


def test_loop_grouped_heads_and_fp32(clm_gpu):
    """Three stage heads (64 streams, 3 steps), and the one-stream fp32 step (5 steps)."""
    _loop_case(clm_gpu, 3, 64, 64, 3)
    _loop_case(clm_gpu, 1, 1, 1, 5, replay=True)


def _fp8_quantize_pool(kp, vp):
    """The bf16 pool (keys [nb, H, bs, D], values [nb, H, D, bs]) quantized row
    by row with the oracle's quantizer into the FP8 cache layouts: keys [nb,
    H, D/8, bs, 8], values [nb, H, D, bs], scales [nb, H, bs].  Slots holding
    NaN (never written) become NaN codes with NaN scales."""
    from oracle import fp8
    out = []
    for rows in (synth.bf16_bits_to_f32(kp), synth.bf16_bits_to_f32(vp).transpose(0, 1, 3, 2)):
        empty = np.isnan(rows).any(axis=-1)
        codes, sc = fp8.quantize_rows(np.where(empty[..., None], 0.0, rows).astype(np.float32))
        codes[empty] = 0x7F
        sc = sc.astype(np.float32)
        sc[empty] = np.nan
        out.append((codes, sc))
    (kc, ks), (vc, vs) = out
    nb, H, bs, D = kc.shape
    kc = np.ascontiguousarray(kc.reshape(nb, H, bs, D // 8, 8).transpose(0, 1, 3, 2, 4))
    return kc, np.ascontiguousarray(vc.transpose(0, 1, 3, 2)), ks, vs


def _fp8_stream_rows(kc, vc, ks, vs, bt, b, n, bs):
    """Stream b's first n positions of the FP8 pool, dequantized by the oracle:
    K, V [n, H, D] (pages gathered at once rather than slot by slot)."""
    from oracle import fp8
    nb, H, G8, _, _ = kc.shape
    D = G8 * 8
    pages = bt[b, :(n + bs - 1) // bs]
    kcodes = kc[pages].transpose(0, 3, 1, 2, 4).reshape(-1, H, D)[:n]      # [pos, H, D]
    vcodes = vc[pages].transpose(0, 3, 1, 2).reshape(-1, H, D)[:n]
    ksc = ks[pages].transpose(0, 2, 1).reshape(-1, H)[:n]
    vsc = vs[pages].transpose(0, 2, 1).reshape(-1, H)[:n]
    return fp8.dequantize_rows(kcodes, ksc), fp8.dequantize_rows(vcodes, vsc)


def _fp8_loop_case(clm_gpu, cfg, B_live, n_steps, rope=False):
    """The loop over an FP8 (E4M3) cache: every step's quantizing append
    against the oracle's quantizer (the whole cache bit for bit at the end),
    attention, logits and tokens against the oracle on the dequantized rows,
    following the oracle's own decisions."""
    import torch
    from oracle import fp8
    x = synth.make_inputs(cfg, B=B_live)
    c = x.cfg
    bs, Kq, Hk, Hq, D, V = c.block_size, c.Kq, c.H_kv, c.H_q, c.D, c.V
    f32 = x.f32
    kp, vp, bt, nb = x.pool_with_room((n_steps - 1) * Kq)
    kc, vc, ks, vs = _fp8_quantize_pool(kp, vp)
    steps = [x.step_arrays(s) for s in range(n_steps)]
    T = lambda a, b16=False: to_torch(np.ascontiguousarray(a), bf16=b16)
    lb0 = x.len_before.astype(np.int32)
    g = dict(k_cache=T(kc), v_cache=T(vc), k_scale=T(ks), v_scale=T(vs), block_table=T(bt), len_before=T(lb0),
             kv_len=T(lb0 + Kq), k_new=T(np.stack([k for k, _, _ in steps]), True),
             v_new=T(np.stack([v for _, v, _ in steps]), True), q=T(np.stack([q for _, _, q in steps]), True),
             W=T(x.W, True))
    dev = torch.device("cuda")
    g["o"] = torch.empty_like(g["q"])
    g["logits"] = torch.empty((n_steps, c.M, V), dtype=torch.float32, device=dev)
    spec_np = None
    if c.mode == "spec":
        spec_np = [x.spec_inputs(s) for s in range(n_steps)]
        for k in ("draft_probs", "draft_tokens", "u_accept", "u_resample"):
            g[k] = T(np.stack([sp[k] for sp in spec_np]))
        g["out_tokens"] = torch.empty((n_steps, c.B, Kq), dtype=torch.int32, device=dev)
        g["num_emitted"] = torch.empty((n_steps, c.B), dtype=torch.int32, device=dev)
    else:
        g["tokens"] = torch.empty((n_steps, c.M), dtype=torch.int32, device=dev)
    max_kv = int((lb0 + n_steps * Kq).max())
    need_ws = clm_gpu.decode_attention_workspace_size(c.B, Kq, Hq, Hk, D, max_kv)
    ws = torch.empty(need_ws + 256, dtype=torch.uint8, device=dev)
    ws = ws[(-ws.data_ptr()) % 256:]
    offset = 1000
    if rope:
        g["positions"] = T((lb0[:, None] + offset + np.arange(Kq)[None, :]).astype(np.int32))
    loop = clm_gpu.DecodeLoop(max_kv_len=max_kv, mode=c.mode, spec_temperature=c.temperature, attn_workspace=ws,
                              block_size=bs, rope_base=1.0e6, **g)
    loop.launch()
    torch.cuda.synchronize()

    scale = 1.0 / math.sqrt(D)
    lb = x.len_before.astype(np.int64).copy()
    live = np.ones(c.B, bool)
    Wf = f32(x.W)
    for s in range(n_steps):
        kn, vn, qs = steps[s]
        kf, qf = f32(kn), f32(qs)
        if rope:            # keys quantized from their fp32 rotation; the rotated queries are stored as bf16
            pos = lb[:, None] + offset + np.arange(Kq)[None, :]
            kf = oracle.rope(kf, pos[:, :, None], 1.0e6).astype(np.float32)
            qf = oracle.round_to_bf16(oracle.rope(qf, pos[:, :, None], 1.0e6)).astype(np.float32)
        kc, vc, ks, vs = fp8.fp8_kv_cache_append(kc, vc, ks, vs, bt, lb.astype(np.int32), kf, f32(vn), bs)
        kv_len = (lb + Kq).astype(np.int32)
        rows_kv = [_fp8_stream_rows(kc, vc, ks, vs, bt, b, int(kv_len[b]), bs) for b in range(c.B)]
        sp = spec_np[s] if spec_np else None
        ref = oracle.decode_step(qf, [r[0] for r in rows_kv], [r[1] for r in rows_kv], kv_len, scale, Hk, Wf,
                                 None, True, mode=c.mode,
                                 temperature=c.temperature if c.mode == "spec" else None, spec=sp)
        sel = np.nonzero(live)[0]
        rows = (sel[:, None] * Kq + np.arange(Kq)[None, :]).reshape(-1)
        check_close(bf16_tensor_to_f32(g["o"][s])[sel], ref["o"][sel], f"fp8 loop c{cfg} step {s} attention")
        check_close(g["logits"][s].cpu().numpy()[rows], ref["logits"][rows], f"fp8 loop c{cfg} step {s} logits")
        if c.mode == "spec":
            ot, ne = g["out_tokens"][s].cpu().numpy(), g["num_emitted"][s].cpu().numpy()
            check_verify(ot[sel], ne[sel], ref["logits"].reshape(c.B, Kq, V)[sel], sp["draft_probs"][sel],
                         sp["draft_tokens"][sel], sp["u_accept"][sel], sp["u_resample"][sel], c.temperature,
                         f"fp8 loop c{cfg} step {s} verify")
            add = ref["num_emitted"].astype(np.int64)
            for b in sel:
                if ne[b] != add[b] or not np.array_equal(ot[b], ref["out_tokens"][b]):
                    live[b] = False
        else:
            check_argmax(g["tokens"][s].cpu().numpy()[rows], ref["logits"][rows], f"fp8 loop c{cfg} step {s} argmax")
            add = np.full(c.B, Kq, np.int64)
        lb = lb + add
    assert np.array_equal(g["len_before"].cpu().numpy()[live], lb[live]), "lengths after the loop"
    if rope:
        assert np.array_equal(g["positions"].cpu().numpy()[live],
                              (lb[:, None] + offset + np.arange(Kq)[None, :])[live])
    elif live.all():        # with rotary the keys' codes may sit one step apart at rounding boundaries
        blocks = np.unique(bt)
        np.testing.assert_array_equal(g["k_cache"].cpu().numpy()[blocks], kc[blocks], err_msg="fp8 key codes")
        np.testing.assert_array_equal(g["v_cache"].cpu().numpy()[blocks], vc[blocks], err_msg="fp8 value codes")
        for name, ref_sc in (("k_scale", ks), ("v_scale", vs)):
            np.testing.assert_array_equal(g[name].cpu().numpy()[blocks].view(np.uint32),
                                          ref_sc[blocks].view(np.uint32), err_msg=f"fp8 {name}")
    loop.close()
    print(f"fp8 loop c{cfg}: {n_steps} steps, {c.B} streams, {int((~live).sum())} parted on exempt decisions")


def test_loop_fp8_cache(clm_gpu):
    """FP8 cache in the loop: 24 streams of the 256-stream mix, greedy, 3
    steps (one or two query rows per KV head), and the 6-query blocks with
    verification, 3 steps (12 rows)."""
    _fp8_loop_case(clm_gpu, 5, 24, 3)
    _fp8_loop_case(clm_gpu, 4, 32, 3)


def test_loop_fp8_cache_rope(clm_gpu):
    """FP8 cache with rotary positions in the loop (the rotary FP8 append):
    24 streams of the 256-stream mix, greedy, and the 6-query blocks with
    verification, 3 steps each; positions advance with the lengths."""
    _fp8_loop_case(clm_gpu, 5, 24, 3, rope=True)
    _fp8_loop_case(clm_gpu, 4, 32, 3, rope=True)
