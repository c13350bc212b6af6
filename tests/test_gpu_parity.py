"""GPU parity: each C-ABI call, and the chained step, against the oracle.

All inputs come from synth (seeded); every expected value comes from oracle/.
Sizes: the five workloads at full size except the 256-stream one, which runs
with its first 24 streams here and at full size (sampled streams checked) in
test_full_size_high_concurrency.
"""

import math
import sys

import numpy as np
import pytest

import oracle
import synth
from parity import (bf16_tensor_to_f32, tolerance_used, check_argmax, check_close, check_sampled, check_verify,
                    to_torch)

pytestmark = pytest.mark.gpu

SMALL_B = {1: None, 2: None, 3: None, 4: None, 5: 24}
_CACHE = {}


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield


def inputs(cfg_index, B=None):
    key = (cfg_index, B)
    if key not in _CACHE:
        _CACHE.clear()
        _CACHE[key] = synth.make_inputs(cfg_index, B=B)
    return _CACHE[key]


class Dev:
    """The step's arrays on the GPU."""

    def __init__(self, x, include_new):
        import torch
        bf = x.cfg.dtype == "bf16"
        self.bf = bf
        kp, vp = x.build_pool(include_new=include_new)
        self.k_pool_host, self.v_pool_host = kp, vp
        self.k_cache = to_torch(kp, bf16=bf)
        self.v_cache = to_torch(vp, bf16=bf)
        self.block_table = to_torch(x.block_table)
        self.kv_len = to_torch(x.kv_len)
        self.len_before = to_torch(x.len_before)
        self.k_new = to_torch(x.k_new, bf16=bf)
        self.v_new = to_torch(x.v_new, bf16=bf)
        self.q = to_torch(x.q, bf16=bf)
        self.W = to_torch(x.W, bf16=bf)
        self.head_id = to_torch(x.head_id) if x.cfg.G > 1 else None
        self.max_kv_len = int(x.kv_len.max())
        torch.cuda.synchronize()


def logical(x):
    return [x.logical_k(b) for b in range(x.cfg.B)], [x.logical_v(b) for b in range(x.cfg.B)]


def as_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_kv_append_bit_exact(clm_gpu, cfg):
    x = inputs(cfg, SMALL_B[cfg])
    d = Dev(x, include_new=False)
    clm_gpu.kv_cache_append(d.k_new, d.v_new, d.k_cache, d.v_cache, d.block_table, d.len_before,
                            block_size=x.cfg.block_size)
    rk, rv = oracle.kv_cache_append(d.k_pool_host, d.v_pool_host, x.block_table, x.len_before,
                                    x.k_new, x.v_new, x.cfg.block_size)
    gk, gv = as_bits(d.k_cache), as_bits(d.v_cache)
    dt = np.int16 if d.bf else np.uint32
    np.testing.assert_array_equal(gk, rk.view(dt))
    np.testing.assert_array_equal(gv, rv.view(dt))


@pytest.mark.parametrize("cfg,offset", [(1, 0), (2, 1000), (4, 37), (5, 123456)])
def test_rope_kv_append(clm_gpu, cfg, offset):
    """Fused rotary append at logical positions len_before + offset + t: the
    rotated new keys in their slots and the rotated queries against the
    oracle; values and every other slot bit-exact."""
    import torch
    x = inputs(cfg, SMALL_B[cfg])
    c = x.cfg
    bf = c.dtype == "bf16"
    d = Dev(x, include_new=False)
    pos = (x.len_before[:, None] + offset + np.arange(c.Kq)[None, :]).astype(np.int32)
    base = 1.0e6
    q = d.q.clone()
    before_k, before_v = as_bits(d.k_cache), as_bits(d.v_cache)
    clm_gpu.rope_kv_cache_append(q, d.k_new, d.v_new, d.k_cache, d.v_cache, d.block_table, d.len_before,
                                 to_torch(pos), base, block_size=c.block_size)
    kp, vp = x.build_pool(include_new=False)
    f32 = (lambda a: synth.bf16_bits_to_f32(a)) if bf else (lambda a: a)
    q_ref, k_ref, _ = oracle.rope_kv_cache_append(f32(x.q), f32(kp), f32(vp), x.block_table, x.len_before,
                                                  pos, f32(x.k_new), f32(x.v_new), c.block_size, base)
    check_close(bf16_tensor_to_f32(q), q_ref, f"rope q c{cfg}")
    # the new rows, gathered through the block table
    k_gpu = bf16_tensor_to_f32(d.k_cache)
    for b in range(c.B):
        for t in range(c.Kq):
            p_ = int(x.len_before[b]) + t
            blk, slot = int(x.block_table[b, p_ // c.block_size]), p_ % c.block_size
            check_close(k_gpu[blk, :, slot, :], k_ref[blk, :, slot, :], f"rope k c{cfg} b{b} t{t}")
    # values exactly as the plain append writes them; untouched key slots unchanged
    kp_plain, vp_plain = x.build_pool(include_new=True)
    v_bits = as_bits(d.v_cache)
    np.testing.assert_array_equal(v_bits, as_bits(to_torch(vp_plain, bf16=bf)))
    k_bits = as_bits(d.k_cache)
    touched = np.zeros(k_bits.shape[:1] + k_bits.shape[2:3], bool)     # [nb, bs]
    for b in range(c.B):
        for t in range(c.Kq):
            p_ = int(x.len_before[b]) + t
            touched[int(x.block_table[b, p_ // c.block_size]), p_ % c.block_size] = True
    keep = ~touched
    np.testing.assert_array_equal(k_bits.transpose(0, 2, 1, 3)[keep], before_k.transpose(0, 2, 1, 3)[keep])
    del torch, before_v


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_decode_attention_parity(clm_gpu, cfg):
    x = inputs(cfg, SMALL_B[cfg])
    d = Dev(x, include_new=True)
    scale = 1.0 / math.sqrt(x.cfg.D)
    o = clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, d.block_table, d.kv_len, d.max_kv_len,
                                 scale=scale)
    keys, vals = logical(x)
    ref = oracle.decode_attention(x.f32(x.q), keys, vals, x.kv_len, scale, x.cfg.H_kv)
    err = check_close(bf16_tensor_to_f32(o), ref, f"attention c{cfg}")
    print(f"attention c{cfg}: max abs err {err:.3g}")
    # run-to-run determinism
    o2 = clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, d.block_table, d.kv_len, d.max_kv_len,
                                  scale=scale)
    assert np.array_equal(as_bits(o), as_bits(o2))



def test_decode_attention_multi_query_many_streams(clm_gpu):
    """Blocks of 6 queries over more than 512 streams: the register-staged
    matrix-core kernel (the LDS-staged one takes up to 512).  520 streams of
    6..70 keys, bf16 N(0, 1) keys and values in a shuffled page pool; every
    13th stream is checked against the oracle."""
    rng = np.random.default_rng(5206)
    B, Kq, Hq, Hk, D, bs = 520, 6, 16, 8, 128, 16
    kv_len = rng.integers(Kq, 71, size=B).astype(np.int32)
    pages = (kv_len + bs - 1) // bs
    nb = int(pages.sum()) + 2
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.zeros((B, int(pages.max())), np.int32)
    o_ = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[o_:o_ + pages[b]]
        o_ += pages[b]
    kc = synth.f32_to_bf16_bits(rng.standard_normal((nb, Hk, bs, D)).astype(np.float32))
    vc = synth.f32_to_bf16_bits(rng.standard_normal((nb, Hk, D, bs)).astype(np.float32))
    q = synth.f32_to_bf16_bits(rng.standard_normal((B, Kq, Hq, D)).astype(np.float32))
    scale = 1.0 / math.sqrt(D)
    o = clm_gpu.decode_attention(to_torch(q, bf16=True), to_torch(kc, bf16=True), to_torch(vc, bf16=True),
                                 to_torch(bt), to_torch(kv_len), int(kv_len.max()), scale=scale)
    idx = np.arange(0, B, 13)
    kf, vf = synth.bf16_bits_to_f32(kc), synth.bf16_bits_to_f32(vc)
    keys, vals = {}, {}
    for b in idx:
        pos = np.arange(int(kv_len[b]))
        blk, slot = bt[b, pos // bs], pos % bs
        keys[b] = kf[blk, :, slot, :]          # [n, H_kv, D]
        vals[b] = vf[blk, :, :, slot]          # [n, H_kv, D]
    ref = oracle.decode_attention(synth.bf16_bits_to_f32(q), keys, vals, kv_len, scale, Hk, streams=idx)
    check_close(bf16_tensor_to_f32(o)[idx], ref[idx], "6-query attention, 520 streams (sampled)")


def _random_pool_case(rng, kv_len, Kq, Hq, Hk, D, bs):
    """bf16 N(0, 1) keys, values and queries for streams of the given lengths in
    a shuffled page pool.  Returns the host arrays and the logical per-stream
    K, V (float32) the oracle reads."""
    kv_len = np.asarray(kv_len, np.int32)
    B = kv_len.size
    pages = (kv_len + bs - 1) // bs
    nb = int(pages.sum()) + 2
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.zeros((B, int(pages.max())), np.int32)
    o_ = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[o_:o_ + pages[b]]
        o_ += pages[b]
    kc = synth.f32_to_bf16_bits(rng.standard_normal((nb, Hk, bs, D), dtype=np.float32))
    vc = synth.f32_to_bf16_bits(rng.standard_normal((nb, Hk, D, bs), dtype=np.float32))
    q = synth.f32_to_bf16_bits(rng.standard_normal((B, Kq, Hq, D), dtype=np.float32))
    kf, vf = synth.bf16_bits_to_f32(kc), synth.bf16_bits_to_f32(vc)
    keys, vals = [], []
    for b in range(B):
        pos = np.arange(int(kv_len[b]))
        blk, slot = bt[b, pos // bs], pos % bs
        keys.append(kf[blk, :, slot, :])       # [n, H_kv, D]
        vals.append(vf[blk, :, :, slot])       # [n, H_kv, D]
    return kv_len, bt, kc, vc, q, keys, vals


def test_decode_attention_max_streams(clm_gpu):
    """The largest batch a call takes: 4096 streams (B * H_kv = 32768) of 1..48
    keys, one query each; every stream against the oracle."""
    rng = np.random.default_rng(4096)
    Hq, Hk, D, bs = 16, 8, 128, 16
    kv_len, bt, kc, vc, q, keys, vals = _random_pool_case(rng, rng.integers(1, 49, size=4096), 1, Hq, Hk, D, bs)
    scale = 1.0 / math.sqrt(D)
    o = clm_gpu.decode_attention(to_torch(q, bf16=True), to_torch(kc, bf16=True), to_torch(vc, bf16=True),
                                 to_torch(bt), to_torch(kv_len), int(kv_len.max()), scale=scale)
    ref = oracle.decode_attention(synth.bf16_bits_to_f32(q), keys, vals, kv_len, scale, Hk)
    check_close(bf16_tensor_to_f32(o), ref, "attention, 4096 streams")


@pytest.mark.parametrize("Kq", [1, 6])
def test_decode_attention_split_boundaries(clm_gpu, Kq):
    """Lengths on and next to multiples of the split and of the 16-token tile:
    12 streams with a bound of 129 keys take 64-token splits under both rules
    (one query: the vector kernel; 6-query blocks: the matrix-core kernel), so
    streams end one before, on and one after the first and second split
    boundaries, where the last split is full, short or a single key."""
    rng = np.random.default_rng(64 + Kq)
    Hq, Hk, D, bs = 16, 8, 128, 16
    lens = [max(Kq, 1), 15, 16, 17, 63, 64, 65, 127, 128, 129, 32, 48 if Kq == 1 else 70]
    kv_len, bt, kc, vc, q, keys, vals = _random_pool_case(rng, lens, Kq, Hq, Hk, D, bs)
    scale = 1.0 / math.sqrt(D)
    rows = 2 if Kq == 1 else 12                 # query rows per KV head, as the kernels pad them
    assert clm_gpu.decode_attention_workspace_size(12, Kq, Hq, Hk, D, 129) == 12 * Hk * 3 * rows * (2 + D) * 4, \
        "partials for 3 splits of 64 tokens per stream"
    o = clm_gpu.decode_attention(to_torch(q, bf16=True), to_torch(kc, bf16=True), to_torch(vc, bf16=True),
                                 to_torch(bt), to_torch(kv_len), 129, scale=scale)
    ref = oracle.decode_attention(synth.bf16_bits_to_f32(q), keys, vals, kv_len, scale, Hk)
    check_close(bf16_tensor_to_f32(o), ref, f"attention at split boundaries, Kq={Kq}")


def test_decode_attention_long_context(clm_gpu):
    """One stream of 100,000 keys next to one of a single key: 98 splits of
    1024 tokens for the long stream, so the merge pass combines more splits
    than one wave has lanes (two passes over the split partials)."""
    rng = np.random.default_rng(100000)
    Hq, Hk, D, bs = 16, 8, 128, 16
    kv_len, bt, kc, vc, q, keys, vals = _random_pool_case(rng, [100000, 1], 1, Hq, Hk, D, bs)
    scale = 1.0 / math.sqrt(D)
    o = clm_gpu.decode_attention(to_torch(q, bf16=True), to_torch(kc, bf16=True), to_torch(vc, bf16=True),
                                 to_torch(bt), to_torch(kv_len), 100000, scale=scale)
    ref = oracle.decode_attention(synth.bf16_bits_to_f32(q), keys, vals, kv_len, scale, Hk)
    check_close(bf16_tensor_to_f32(o), ref, "attention, 100,000 keys")


def test_decode_attention_shortest_blocks(clm_gpu):
    """6-query causal blocks whose first query sees a single key (kv_len = Kq)
    and blocks of every length up to two tiles, on the LDS-staged
    matrix-core kernel."""
    rng = np.random.default_rng(606)
    Kq, Hq, Hk, D, bs = 6, 16, 8, 128, 16
    lens = np.concatenate([np.full(8, Kq), np.arange(Kq, 40)])
    kv_len, bt, kc, vc, q, keys, vals = _random_pool_case(rng, lens, Kq, Hq, Hk, D, bs)
    scale = 1.0 / math.sqrt(D)
    o = clm_gpu.decode_attention(to_torch(q, bf16=True), to_torch(kc, bf16=True), to_torch(vc, bf16=True),
                                 to_torch(bt), to_torch(kv_len), int(kv_len.max()), scale=scale)
    ref = oracle.decode_attention(synth.bf16_bits_to_f32(q), keys, vals, kv_len, scale, Hk)
    check_close(bf16_tensor_to_f32(o), ref, "6-query attention, shortest blocks")


@pytest.mark.parametrize("cfg,bs,B,D", [(2, 32, None, 128), (3, 64, 16, 128), (4, 32, None, 128), (4, 128, 12, 128),
                                        (2, 16, None, 64), (4, 16, None, 64), (4, 32, 12, 64),
                                        (4, 128, 16, 128), (2, 128, 8, 128)])
def test_block_sizes(clm_gpu, cfg, bs, B, D):
    """Pages of 16 to 128 slots and head widths 128 and 64 (the block-size-
    generic kernels and the D = 64 instantiations): the append bit-exact, then
    attention over the cache it wrote, against the oracle.  Single-query rows
    take the vector kernel; the 6-query blocks the matrix-core kernel with its
    LDS ring.  The last two cases start splits inside a page: 192-token
    splits over 128-slot pages (16 x 6-query blocks) and 64-token splits over
    128-slot pages (8 single-query streams)."""
    import dataclasses
    c = dataclasses.replace(synth.get_config(cfg), block_size=bs, D=D)
    x = synth.make_inputs(c, B=B)
    d = Dev(x, include_new=False)
    clm_gpu.kv_cache_append(d.k_new, d.v_new, d.k_cache, d.v_cache, d.block_table, d.len_before, block_size=bs)
    rk, rv = oracle.kv_cache_append(d.k_pool_host, d.v_pool_host, x.block_table, x.len_before,
                                    x.k_new, x.v_new, bs)
    dt = np.int16 if d.bf else np.uint32
    np.testing.assert_array_equal(as_bits(d.k_cache), rk.view(dt))
    np.testing.assert_array_equal(as_bits(d.v_cache), rv.view(dt))
    scale = 1.0 / math.sqrt(x.cfg.D)
    o = clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, d.block_table, d.kv_len, d.max_kv_len, scale=scale,
                                 block_size=bs)
    keys, vals = logical(x)
    ref = oracle.decode_attention(x.f32(x.q), keys, vals, x.kv_len, scale, x.cfg.H_kv)
    check_close(bf16_tensor_to_f32(o), ref, f"attention c{cfg} block size {bs} D {D}")

@pytest.mark.parametrize("cfg", [2, 5])
def test_decode_attention_split_plan_and_batch_order(clm_gpu, cfg):
    """A looser max_kv_len bound changes the split plan (longer splits, more
    of them per stream); permuting streams must not change any stream's
    output bits."""
    import torch
    x = inputs(cfg, SMALL_B[cfg])
    d = Dev(x, include_new=True)
    scale = 1.0 / math.sqrt(x.cfg.D)
    o = clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, d.block_table, d.kv_len, d.max_kv_len, scale=scale)
    loose = 3 * d.max_kv_len
    assert clm_gpu.decode_attention_workspace_size(x.cfg.B, 1, 16, 8, 128, loose) != \
        clm_gpu.decode_attention_workspace_size(x.cfg.B, 1, 16, 8, 128, d.max_kv_len)
    o_big = clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, d.block_table, d.kv_len, loose, scale=scale)
    check_close(bf16_tensor_to_f32(o_big), bf16_tensor_to_f32(o), f"split plan c{cfg}", atol=1e-2, rtol=1e-2)
    perm = torch.randperm(x.cfg.B, generator=torch.Generator().manual_seed(7)).to(d.q.device)
    o_p = clm_gpu.decode_attention(d.q[perm].contiguous(), d.k_cache, d.v_cache, d.block_table[perm].contiguous(),
                                   d.kv_len[perm].contiguous(), d.max_kv_len, scale=scale)
    assert np.array_equal(as_bits(o_p), as_bits(o[perm].contiguous()))


def test_decode_attention_workspace_reuse_across_shapes(clm_gpu):
    """One workspace serves calls of different batch sizes in turn; a call
    must not depend on what an earlier call left in it."""
    import torch
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    outs = {}
    for cfg, B in [(5, 24), (2, None), (5, 24), (3, None), (5, 24)]:
        x = inputs(cfg, B)
        d = Dev(x, include_new=True)
        o = clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, d.block_table, d.kv_len, d.max_kv_len,
                                     workspace=ws)
        if cfg == 5:
            if 5 in outs:
                assert np.array_equal(as_bits(o), outs[5])
            else:
                outs[5] = as_bits(o)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_codebook_head_isolated(clm_gpu, cfg):
    x = inputs(cfg, SMALL_B[cfg])
    bf = x.cfg.dtype == "bf16"
    h = x.h_iso()
    W = to_torch(x.W, bf16=bf)
    hid = to_torch(x.head_id) if x.cfg.G > 1 else None
    logits = clm_gpu.codebook_head(to_torch(h, bf16=bf), W, hid)
    ref = oracle.codebook_head(x.f32(h), x.f32(x.W), x.head_id)
    err = check_close(logits.cpu().numpy(), ref, f"head c{cfg}")
    tok = clm_gpu.sample_or_argmax(logits)
    ex = check_argmax(tok.cpu().numpy(), ref.astype(np.float32), f"head argmax c{cfg}")
    print(f"head c{cfg}: max abs err {err:.3g}, argmax exempt {ex}/{x.cfg.M}")


def test_codebook_head_ragged_rows(clm_gpu):
    """Row counts that are not multiples of 16, 64 or 128, vocabularies that
    are not multiples of the entry tile, several row chunks per head, one head
    holding most rows, heads that get no rows at all (the eight-head limit
    with only the last one used), and d from 128 up."""
    rng = np.random.default_rng(5)
    cases = [(1, 4096, 1, 256), (17, 1000, 1, 256), (70, 4096, 3, 256), (130, 4160, 2, 256),
             (129, 1000, 1, 128), (300, 4160, 1, 384), (260, 20000, 1, 256),
             (300, 4096, 2, 256), (50, 4096, 4, 256), (200, 1000, 8, 128)]
    for M, V, G, d in cases:
        h = synth.f32_to_bf16_bits(rng.standard_normal((M, d)).astype(np.float32))
        W = synth.f32_to_bf16_bits((rng.standard_normal((G, V, d)) * 0.05).astype(np.float32))
        hid = rng.integers(0, G, size=M).astype(np.int32)
        if G == 2 and M == 300:
            hid[:220] = 1                       # one head takes 220 of the rows
        if G == 4:
            hid = np.where(hid < 2, 0, 3).astype(np.int32)      # heads 1 and 2 get no rows
        if G == 8:
            hid[:] = 7                          # all rows on the last of eight heads
        logits = clm_gpu.codebook_head(to_torch(h, bf16=True), to_torch(W, bf16=True),
                                       to_torch(hid) if G > 1 else None)
        ref = oracle.codebook_head(synth.bf16_bits_to_f32(h), synth.bf16_bits_to_f32(W), hid)
        check_close(logits.cpu().numpy(), ref, f"head M={M} V={V} G={G} d={d}")


@pytest.mark.parametrize("M,G,V,d,F", [(16, 1, 16384, 2048, 4096), (64, 3, 4096, 2048, 4096),
                                        (70, 2, 1000, 256, 384), (192, 1, 4096, 2048, 4096)])
def test_codebook_head_mlp(clm_gpu, M, G, V, d, F):
    """TontaubeV1's two-layer head (d -> F -> Mish -> V per stage): the bf16
    activation and the logits against the oracle, including ragged row and
    vocabulary counts and rows of three stages."""
    rng = np.random.default_rng(M + V)
    h = synth.f32_to_bf16_bits(rng.standard_normal((M, d)).astype(np.float32))
    W1 = synth.f32_to_bf16_bits((rng.standard_normal((G, F, d)) * 0.02).astype(np.float32))
    W2 = synth.f32_to_bf16_bits((rng.standard_normal((G, V, F)) * 0.02).astype(np.float32))
    hid = rng.integers(0, G, size=M).astype(np.int32)
    logits, act = clm_gpu.codebook_head_mlp(to_torch(h, bf16=True), to_torch(W1, bf16=True),
                                            to_torch(W2, bf16=True), to_torch(hid) if G > 1 else None)
    ref_act, ref = oracle.codebook_head_mlp(synth.bf16_bits_to_f32(h), synth.bf16_bits_to_f32(W1),
                                            synth.bf16_bits_to_f32(W2), hid)
    check_close(bf16_tensor_to_f32(act), ref_act, f"mlp act M={M} G={G} V={V}")
    err = check_close(logits.cpu().numpy(), ref, f"mlp logits M={M} G={G} V={V}")
    print(f"mlp head M={M} G={G} V={V}: max abs err {err:.3g}")


@pytest.mark.parametrize("cfg,scale", [(2, 1.0), (2, 4.0), (5, 1.0), (3, 1.0)])
def test_sampler_isolated(clm_gpu, cfg, scale):
    import torch
    x = inputs(cfg, SMALL_B[cfg])
    logits = x.logits_iso(scale)
    u = x.uniforms()
    lt = to_torch(logits)
    M = x.cfg.M
    temp = np.full(M, 0.7, np.float32)
    tok = clm_gpu.sample_or_argmax(lt, to_torch(temp), to_torch(u)).cpu().numpy()
    ex = check_sampled(tok, logits, temp, u, f"sample c{cfg} x{scale}")
    greedy = clm_gpu.sample_or_argmax(lt).cpu().numpy()
    ex2 = check_argmax(greedy, logits, f"argmax c{cfg}")
    # per-row mix of greedy and sampled rows, with a vocabulary mask
    temp_mix = np.where(np.arange(M) % 2 == 0, 0.0, 0.7).astype(np.float32)
    vv = np.where(np.arange(M) % 3 == 0, x.cfg.V // 2 + 1, x.cfg.V).astype(np.int32)
    mix = clm_gpu.sample_or_argmax(lt, to_torch(temp_mix), to_torch(u), to_torch(vv)).cpu().numpy()
    for r in range(M):
        if temp_mix[r] == 0:
            check_argmax(mix[r:r + 1], logits[r:r + 1], "mix argmax", vocab_valid=vv[r:r + 1])
        else:
            check_sampled(mix[r:r + 1], logits[r:r + 1], temp_mix[r:r + 1], u[r:r + 1], "mix sample",
                          vocab_valid=vv[r:r + 1])
    print(f"sampler c{cfg} x{scale}: exempt sampled {ex}/{M}, argmax {ex2}/{M}")
    del torch


def test_sampler_closed_forms(clm_gpu):
    """Equal logits give floor(u*V); a one-hot row gives its hot index; u = 0
    gives the first positive-probability token; padded rows (ld > V)."""
    V = 1000
    u = np.array([(k + 0.5) / 10 for k in range(10)], np.float32)
    logits = np.zeros((10, V), np.float32)
    tok = clm_gpu.sample_or_argmax(to_torch(logits), to_torch(np.full(10, 0.7, np.float32)), to_torch(u)).cpu().numpy()
    assert tok.tolist() == [int(ui * V) for ui in u]
    hot = np.full((4, 1024 + 8), -1e30, np.float32)     # exp underflows to exactly 0
    for r in range(4):
        hot[r, 100 * r + 7] = 60.0
    lt = to_torch(hot)[:, :1024]   # padded rows
    t = clm_gpu.sample_or_argmax(lt, to_torch(np.full(4, 1.0, np.float32)),
                                 to_torch(np.array([0.0, 0.3, 0.7, 0.999], np.float32))).cpu().numpy()
    assert t.tolist() == [7, 107, 207, 307]
    y = np.full((1, 4096), -1e30, np.float32)
    y[0, 3000:] = 0.0
    t0 = clm_gpu.sample_or_argmax(to_torch(y), to_torch(np.ones(1, np.float32)), to_torch(np.zeros(1, np.float32)))
    assert int(t0.cpu()[0]) == 3000
    # the largest uniform below 1 takes the last token of positive weight:
    # equal logits (last index), zero weight past index 499, a vocabulary
    # mask at 300, and a row of two passes with zero weight past 20000
    top = np.float32(1.0) - np.float32(2.0 ** -24)
    z = np.zeros((3, 1000), np.float32)
    z[1, 500:] = -1e30
    tz = clm_gpu.sample_or_argmax(to_torch(z), to_torch(np.full(3, 0.7, np.float32)), to_torch(np.full(3, top)),
                                  vocab_valid=to_torch(np.array([1000, 1000, 300], np.int32))).cpu().numpy()
    assert tz.tolist() == [999, 499, 299]
    w = np.zeros((1, 30000), np.float32)
    w[0, 20001:] = -1e30
    tw = clm_gpu.sample_or_argmax(to_torch(w), to_torch(np.ones(1, np.float32)), to_torch(np.full(1, top)))
    assert int(tw.cpu()[0]) == 20000


@pytest.mark.parametrize("V", [16385, 50000, 100003])
def test_sampler_rows_longer_than_one_pass(clm_gpu, V):
    """Vocabularies past one pass of 16,384 entries (2, 4 and 7 passes): every
    pass is totalled, then the one holding u*S is redone.  Sampled rows at
    T 0.7 and 1.5 with and without a vocabulary mask, and greedy rows, against
    the oracle."""
    rng = np.random.default_rng(V)
    M = 8
    logits = (rng.standard_normal((M, V)) * 3.0).astype(np.float32)
    logits[0, V - 1] = 40.0                       # peaked at the very last entry
    u = rng.random(M, dtype=np.float32)
    temp = np.where(np.arange(M) % 2 == 0, 0.7, 1.5).astype(np.float32)
    vv = np.where(np.arange(M) % 3 == 1, V // 3 + 5, V).astype(np.int32)
    lt = to_torch(logits)
    tok = clm_gpu.sample_or_argmax(lt, to_torch(temp), to_torch(u)).cpu().numpy()
    ex = check_sampled(tok, logits, temp, u, f"sample V={V}")
    tok = clm_gpu.sample_or_argmax(lt, to_torch(temp), to_torch(u), to_torch(vv)).cpu().numpy()
    ex += check_sampled(tok, logits, temp, u, f"sample masked V={V}", vocab_valid=vv)
    greedy = clm_gpu.sample_or_argmax(lt, to_torch(np.zeros(M, np.float32)), to_torch(u), to_torch(vv)).cpu().numpy()
    ex2 = check_argmax(greedy, logits, f"argmax masked V={V}", vocab_valid=vv)
    print(f"long rows V={V}: exempt sampled {ex}/{2 * M}, argmax {ex2}/{M}")


@pytest.mark.parametrize("T", [0.7, 0.0])
def test_spec_verify_rows_longer_than_one_pass(clm_gpu, T):
    """Verification over a 40,000-entry vocabulary (3 passes per row), with and
    without the bonus row: target rows N(0, 3), draft rows softmax of N(0, 2)
    logits, drafted tokens drawn from the draft rows."""
    rng = np.random.default_rng(40000 + int(T * 10))
    B, K, V = 6, 4, 40000
    tl = (rng.standard_normal((B, K + 1, V)) * 3.0).astype(np.float32)
    z = rng.standard_normal((B, K, V)) * 2.0
    q = np.exp(z - z.max(axis=-1, keepdims=True))
    q = (q / q.sum(axis=-1, keepdims=True)).astype(np.float32)
    q64 = q.astype(np.float64)
    drafts = np.array([[rng.choice(V, p=q64[b, i] / q64[b, i].sum()) for i in range(K)]
                       for b in range(B)], np.int32)
    ua = rng.random((B, K), dtype=np.float32)
    ur = rng.random(B, dtype=np.float32)
    tl_k = np.ascontiguousarray(tl[:, :K])
    toks, num = clm_gpu.spec_verify(to_torch(tl_k), to_torch(q), to_torch(drafts), to_torch(ua), to_torch(ur), T)
    ex = check_verify(toks.cpu().numpy(), num.cpu().numpy(), tl_k, q, drafts, ua, ur, T, f"verify V={V} T={T}")
    toks, num = clm_gpu.spec_verify_bonus(to_torch(tl), to_torch(q), to_torch(drafts), to_torch(ua), to_torch(ur), T)
    ex += check_verify(toks.cpu().numpy(), num.cpu().numpy(), tl, q, drafts, ua, ur, T, f"verify bonus V={V} T={T}",
                       bonus=True)
    print(f"verify V={V} T={T}: exempt {ex}/{2 * B}")


@pytest.mark.parametrize("K,V", [(16, 4096), (8, 100), (3, 1)])
def test_spec_verify_draft_counts_and_small_vocabularies(clm_gpu, K, V):
    """The most drafts a call takes (16; 15 with the bonus row), a vocabulary
    shorter than one thread's 16 entries per lane group (100), and a single
    token (every draft is token 0), at T 0.7 and 0, against the oracle."""
    rng = np.random.default_rng(K * 1000 + V)
    B = 5
    for T in (0.7, 0.0):
        for bonus in (False, True):
            k = min(K, 15) if bonus else K
            tl = (rng.standard_normal((B, k + (1 if bonus else 0), V)) * 2.0).astype(np.float32)
            z = rng.standard_normal((B, k, V)) * 2.0
            q64 = np.exp(z - z.max(axis=-1, keepdims=True))
            q64 /= q64.sum(axis=-1, keepdims=True)
            q = q64.astype(np.float32)
            drafts = np.array([[rng.choice(V, p=q64[b, i] / q64[b, i].sum()) for i in range(k)] for b in range(B)],
                              np.int32)
            ua = rng.random((B, k), dtype=np.float32)
            ur = rng.random(B, dtype=np.float32)
            f = clm_gpu.spec_verify_bonus if bonus else clm_gpu.spec_verify
            toks, num = f(to_torch(tl), to_torch(q), to_torch(drafts), to_torch(ua), to_torch(ur), T)
            ex = check_verify(toks.cpu().numpy(), num.cpu().numpy(), tl, q, drafts, ua, ur, T,
                              f"verify K={k} V={V} T={T} bonus={bonus}", bonus=bonus)
            print(f"verify K={k} V={V} T={T} bonus={bonus}: exempt {ex}/{B}")


def test_argmax_ties_alignment_and_tails(clm_gpu):
    """Greedy rows whose maximum is planted at two or three positions (the
    lowest must win), rows that are not 16-byte aligned (ld not a multiple of
    4), vocabularies that are not multiples of 4 or shorter than 4, and masks
    that cut between the planted positions."""
    rng = np.random.default_rng(11)
    for V, ld in [(1, 1), (3, 3), (5, 8), (1003, 1003), (4096, 4099), (16384, 16384), (16387, 16388)]:
        M = 9
        x = rng.standard_normal((M, ld)).astype(np.float32)
        for r in range(M):
            pos = rng.choice(V, size=min(3, V), replace=False)
            x[r, pos] = np.float32(10.0 + (r % 2))
        if V >= 8:
            x[0, V - 1] = 50.0                 # maximum in the last entry (scalar tail when V % 4)
            x[1, 0] = 50.0                     # ... and in the first
        lt = to_torch(x)[:, :V]
        got = clm_gpu.sample_or_argmax(lt).cpu().numpy()
        want = [oracle.argmax_token(x[r, :V]) for r in range(M)]
        assert got.tolist() == want, (V, ld, got.tolist(), want)
        vv = rng.integers(1, V + 1, size=M).astype(np.int32)
        got = clm_gpu.sample_or_argmax(lt, to_torch(np.zeros(M, np.float32)), to_torch(np.zeros(M, np.float32)),
                                       to_torch(vv)).cpu().numpy()
        want = [oracle.argmax_token(x[r, :V], vv[r]) for r in range(M)]
        assert got.tolist() == want, (V, ld, "masked", got.tolist(), want)


def _spec_inputs_torch(s):
    return (to_torch(s["draft_probs"]), to_torch(s["draft_tokens"]), to_torch(s["u_accept"]),
            to_torch(s["u_resample"]))


@pytest.mark.parametrize("T", [0.7, 0.0])
def test_spec_verify_isolated(clm_gpu, T):
    x = inputs(4)
    s = x.spec_inputs()
    tl = s["target_logits_iso"]
    dp, dtok, ua, ur = _spec_inputs_torch(s)
    toks, num = clm_gpu.spec_verify(to_torch(tl), dp, dtok, ua, ur, T)
    ex = check_verify(toks.cpu().numpy(), num.cpu().numpy(), tl, s["draft_probs"], s["draft_tokens"],
                      s["u_accept"], s["u_resample"], T, f"verify T={T}")
    print(f"verify T={T}: exempt {ex}/{x.cfg.B}, mean emitted {num.float().mean().item():.3f}")


def test_spec_verify_accepts_when_draft_equals_target(clm_gpu):
    x = inputs(4)
    s = x.spec_inputs()
    tl = s["target_logits_iso"]
    T = 0.7
    q = np.stack([[oracle.target_probs(tl[b, i], T) for i in range(x.cfg.Kq)] for b in range(x.cfg.B)])
    ua = (s["u_accept"] * np.float32(0.999)).astype(np.float32)
    toks, num = clm_gpu.spec_verify(to_torch(tl), to_torch(q.astype(np.float32)), to_torch(s["draft_tokens"]),
                                    to_torch(ua), to_torch(s["u_resample"]), T)
    # GPU and oracle normalisers may differ in the last bit, so p[x]/q can be
    # just under 1; u < 0.999 keeps every decision an accept.
    assert (num.cpu().numpy() == x.cfg.Kq).all()
    assert np.array_equal(toks.cpu().numpy(), s["draft_tokens"])


@pytest.mark.parametrize("T", [0.7, 0.0])
def test_spec_verify_bonus_isolated(clm_gpu, T):
    x = inputs(4)
    s = x.spec_inputs()
    tl = s["target_logits_bonus_iso"]
    dp, dtok, ua, ur = _spec_inputs_torch(s)
    toks, num = clm_gpu.spec_verify_bonus(to_torch(tl), dp, dtok, ua, ur, T)
    ex = check_verify(toks.cpu().numpy(), num.cpu().numpy(), tl, s["draft_probs"], s["draft_tokens"],
                      s["u_accept"], s["u_resample"], T, f"verify bonus T={T}", bonus=True)
    print(f"verify bonus T={T}: exempt {ex}/{x.cfg.B}, mean emitted {num.float().mean().item():.3f}")


@pytest.mark.parametrize("T", [0.7, 0.0])
def test_spec_verify_bonus_after_all_accepts(clm_gpu, T):
    """Drafts equal to the target distribution (T > 0) or to each row's argmax
    (T = 0) are all accepted, so every stream ends with a bonus draw."""
    x = inputs(4)
    s = x.spec_inputs()
    tl = s["target_logits_bonus_iso"]
    K = x.cfg.Kq
    if T > 0:
        q = np.stack([[oracle.target_probs(tl[b, i], T) for i in range(K)] for b in range(x.cfg.B)])
        drafts = s["draft_tokens"]
    else:
        q = np.full((x.cfg.B, K, x.cfg.V), 1.0 / x.cfg.V, np.float32)
        drafts = np.array([[oracle.argmax_token(tl[b, i]) for i in range(K)] for b in range(x.cfg.B)], np.int32)
    ua = (s["u_accept"] * np.float32(0.999)).astype(np.float32)
    toks, num = clm_gpu.spec_verify_bonus(to_torch(tl), to_torch(q.astype(np.float32)), to_torch(drafts),
                                          to_torch(ua), to_torch(s["u_resample"]), T)
    num = num.cpu().numpy()
    assert (num == K + 1).all()
    ex = check_verify(toks.cpu().numpy(), num, tl, q.astype(np.float32), drafts, ua, s["u_resample"], T,
                      f"bonus all-accept T={T}", bonus=True)
    print(f"bonus all-accept T={T}: exempt {ex}/{x.cfg.B}")


@pytest.mark.parametrize("bonus", [False, True])
def test_spec_verify_first_rejection_at_every_position(clm_gpu, bonus):
    """Stream b's first rejection is planted at draft b % (K+1) (K+1: none):
    drafts before it come from the target distribution itself (ratio 1,
    accepted at u < 0.999), the rejected draft has all its draft mass on one
    token (ratio p(x) << u = 0.5).  Every stream must emit exactly its
    accepted drafts and one residual token; the bonus variant adds a bonus
    token only after K accepts, also when the rejection is at the last draft."""
    x = inputs(4)
    s = x.spec_inputs()
    tl = s["target_logits_bonus_iso"]
    B, K, V, T = x.cfg.B, x.cfg.Kq, x.cfg.V, 0.7
    if not bonus:
        tl = np.ascontiguousarray(tl[:, :K])
    q = np.stack([[oracle.target_probs(tl[b, i], T) for i in range(K)] for b in range(B)]).astype(np.float32)
    drafts = s["draft_tokens"].copy()
    ua = (s["u_accept"] * np.float32(0.999)).astype(np.float32)
    first_rej = np.arange(B) % (K + 1)
    for b in range(B):
        j = int(first_rej[b])
        if j < K:
            q[b, j] = 0.0
            q[b, j, drafts[b, j]] = 1.0
            ua[b, j] = 0.5
    f = clm_gpu.spec_verify_bonus if bonus else clm_gpu.spec_verify
    toks, num = f(to_torch(tl), to_torch(q), to_torch(drafts), to_torch(ua), to_torch(s["u_resample"]), T)
    toks, num = toks.cpu().numpy(), num.cpu().numpy()
    want = np.where(first_rej < K, first_rej + 1, K + (1 if bonus else 0))
    np.testing.assert_array_equal(num, want)
    for b in range(B):
        j = int(first_rej[b])
        np.testing.assert_array_equal(toks[b, :min(j, K)], drafts[b, :min(j, K)])
        assert np.all(toks[b, num[b]:] == -1)
    ex = check_verify(toks, num, tl, q, drafts, ua, s["u_resample"], T, f"planted rejections bonus={bonus}",
                      bonus=bonus)
    print(f"planted rejections bonus={bonus}: exempt {ex}/{B}")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_chained_step(clm_gpu, cfg):
    """append -> attention -> head -> sample/argmax/verify on the GPU, against
    the oracle's chained step."""
    import torch
    x = inputs(cfg, SMALL_B[cfg])
    c = x.cfg
    d = Dev(x, include_new=False)
    scale = 1.0 / math.sqrt(c.D)
    clm_gpu.kv_cache_append(d.k_new, d.v_new, d.k_cache, d.v_cache, d.block_table, d.len_before,
                            block_size=c.block_size)
    o = clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, d.block_table, d.kv_len, d.max_kv_len, scale=scale)
    h = o.view(c.M, c.d_model)
    logits = clm_gpu.codebook_head(h, d.W, d.head_id)
    keys, vals = logical(x)
    spec = x.spec_inputs() if c.mode == "spec" else None
    temp = np.full(c.M, c.temperature, np.float32) if c.mode == "sample" else None
    u = x.uniforms() if c.mode == "sample" else None
    ref = oracle.decode_step(x.f32(x.q), keys, vals, x.kv_len, scale, c.H_kv, x.f32(x.W), x.head_id,
                             c.dtype == "bf16", mode=c.mode,
                             temperature=(c.temperature if c.mode == "spec" else temp), uniforms=u, spec=spec)
    o_f = bf16_tensor_to_f32(o)
    l_f = logits.cpu().numpy()
    err_o = check_close(o_f, ref["o"], f"chained attention c{cfg}")
    err_l = check_close(l_f, ref["logits"], f"chained logits c{cfg}")
    use_o, use_l = tolerance_used(o_f, ref["o"]), tolerance_used(l_f, ref["logits"])
    if c.mode == "spec":
        dp, dtok, ua, ur = _spec_inputs_torch(spec)
        toks, num = clm_gpu.spec_verify(logits.view(c.B, c.Kq, c.V), dp, dtok, ua, ur, c.temperature)
        ex = check_verify(toks.cpu().numpy(), num.cpu().numpy(), ref["logits"].reshape(c.B, c.Kq, c.V),
                          spec["draft_probs"], spec["draft_tokens"], spec["u_accept"], spec["u_resample"],
                          c.temperature, f"chained verify c{cfg}")
    elif c.mode == "sample":
        tok = clm_gpu.sample_or_argmax(logits, to_torch(temp), to_torch(u)).cpu().numpy()
        ex = check_sampled(tok, ref["logits"], temp, u, f"chained sample c{cfg}")
    else:
        tok = clm_gpu.sample_or_argmax(logits).cpu().numpy()
        ex = check_argmax(tok, ref["logits"], f"chained argmax c{cfg}")
    print(f"chained c{cfg} (B {c.B}): max |o err| {err_o:.3g} ({use_o:.2f} of the bar), "
          f"max |logit err| {err_l:.3g} ({use_l:.2f} of the bar), exempt {ex}")
    del torch


def test_tiny_workload_many_draws(clm_gpu):
    """The tiny fp32 workload over 200 independent draws (its greedy tokens
    often sit within the 1e-3 top-2 gap of the argmax rule, so one draw says
    little): the chained step against the oracle's on every draw."""
    import dataclasses
    base = synth.get_config(1)
    exempt = 0
    worst_o = worst_l = 0.0
    for t in range(200):
        x = synth.make_inputs(dataclasses.replace(base, trial=t))
        c = x.cfg
        d = Dev(x, include_new=False)
        scale = 1.0 / math.sqrt(c.D)
        clm_gpu.kv_cache_append(d.k_new, d.v_new, d.k_cache, d.v_cache, d.block_table, d.len_before,
                                block_size=c.block_size)
        o = clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, d.block_table, d.kv_len, d.max_kv_len,
                                     scale=scale)
        logits = clm_gpu.codebook_head(o.view(c.M, c.d_model), d.W)
        tok = clm_gpu.sample_or_argmax(logits).cpu().numpy()
        keys, vals = logical(x)
        ref = oracle.decode_step(x.f32(x.q), keys, vals, x.kv_len, scale, c.H_kv, x.f32(x.W), None, False)
        o_f = o.cpu().numpy()
        l_f = logits.cpu().numpy()
        check_close(o_f, ref["o"], f"tiny attention, draw {t}")
        check_close(l_f, ref["logits"], f"tiny logits, draw {t}")
        worst_o = max(worst_o, tolerance_used(o_f, ref["o"]))
        worst_l = max(worst_l, tolerance_used(l_f, ref["logits"]))
        exempt += check_argmax(tok, ref["logits"], f"tiny argmax, draw {t}")
    print(f"tiny workload, 200 draws: worst {worst_o:.2g} (o) and {worst_l:.2g} (logits) of the bar, "
          f"argmax exempt {exempt}/200")


def test_full_size_high_concurrency(clm_gpu):
    """256 streams, log-uniform KV lengths 64..8192, head 2048->16384, greedy:
    the launch configuration the benchmark times.  Every stream's attention
    output, logits and argmax token against the oracle, and the whole pool
    after the append bit for bit."""
    x = synth.make_inputs(5)
    c = x.cfg
    d = Dev(x, include_new=False)
    scale = 1.0 / math.sqrt(c.D)
    clm_gpu.kv_cache_append(d.k_new, d.v_new, d.k_cache, d.v_cache, d.block_table, d.len_before)
    o = clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, d.block_table, d.kv_len, d.max_kv_len, scale=scale)
    logits = clm_gpu.codebook_head(o.view(c.M, c.d_model), d.W)
    tok = clm_gpu.sample_or_argmax(logits).cpu().numpy()
    keys, vals = logical(x)
    ref = oracle.decode_step(x.f32(x.q), keys, vals, x.kv_len, scale, c.H_kv, x.f32(x.W), None, True)
    o_f = bf16_tensor_to_f32(o)
    l_f = logits.cpu().numpy()
    err_o = check_close(o_f, ref["o"], "full-size attention, all 256 streams")
    err_l = check_close(l_f, ref["logits"], "full-size logits, all 256 streams")
    ex = check_argmax(tok, ref["logits"], "full-size argmax, all 256 streams")
    print(f"full size: max |o err| {err_o:.3g} ({tolerance_used(o_f, ref['o']):.2f} of the bar), "
          f"max |logit err| {err_l:.3g} ({tolerance_used(l_f, ref['logits']):.2f} of the bar), "
          f"argmax exempt {ex}/{c.M}")
    # the append at full size: the whole pool against the oracle's append
    rk, rv = oracle.kv_cache_append(d.k_pool_host, d.v_pool_host, x.block_table, x.len_before,
                                    x.k_new, x.v_new, c.block_size)
    np.testing.assert_array_equal(as_bits(d.k_cache), rk.view(np.int16))
    np.testing.assert_array_equal(as_bits(d.v_cache), rv.view(np.int16))


def test_append_partitions_bit_identical(clm_gpu):
    """The cache after T single-row appends (len_before + t, t = 0..T-1) is
    bit-identical to the cache after one T-row append, and both equal the
    oracle's, on the 6-query workload; likewise split 2 + 4 and 3 + 3."""
    x = inputs(4)
    c = x.cfg
    T = c.Kq
    ref_k, ref_v = oracle.kv_cache_append(*x.build_pool(include_new=False), x.block_table, x.len_before,
                                          x.k_new, x.v_new, c.block_size)
    for parts in ([T], [1] * T, [2, 4], [3, 3]):
        d = Dev(x, include_new=False)
        t0 = 0
        for n in parts:
            lb = to_torch((x.len_before + t0).astype(np.int32))
            clm_gpu.kv_cache_append(d.k_new[:, t0:t0 + n].contiguous(), d.v_new[:, t0:t0 + n].contiguous(),
                                    d.k_cache, d.v_cache, d.block_table, lb, block_size=c.block_size)
            t0 += n
        np.testing.assert_array_equal(as_bits(d.k_cache), ref_k.view(np.int16), err_msg=str(parts))
        np.testing.assert_array_equal(as_bits(d.v_cache), ref_v.view(np.int16), err_msg=str(parts))


@pytest.mark.parametrize("cfg,sub", [(5, 100), (4, 28)])
def test_batch_compaction_bit_identical(clm_gpu, cfg, sub):
    """Dropping streams from a batch (a serving engine compacting finished or
    cancelled streams away) leaves every remaining stream's attention output,
    logits and token bits unchanged.  The attention split length depends on
    streams x KV heads x max_kv_len; it is the same for the full and the
    compacted batch here (1024 tokens for the 256-stream mix and its 100-stream
    subset, 384 for the 32 x 6-query batch and its 28-stream subset), and the
    head's arithmetic does not depend on the row count.  The subset keeps the
    streams in a shuffled order."""
    import torch
    x = inputs(cfg)
    c = x.cfg
    d = Dev(x, include_new=True)
    scale = 1.0 / math.sqrt(c.D)
    spec = x.spec_inputs() if c.mode == "spec" else None

    def run(sel):
        idx = torch.from_numpy(np.asarray(sel, np.int64)).to(d.q.device)
        q = d.q[idx].contiguous()
        o = clm_gpu.decode_attention(q, d.k_cache, d.v_cache, d.block_table[idx].contiguous(),
                                     d.kv_len[idx].contiguous(), d.max_kv_len, scale=scale)
        lg = clm_gpu.codebook_head(o.view(len(sel) * c.Kq, c.d_model), d.W,
                                   None if d.head_id is None else d.head_id.view(c.B, c.Kq)[idx].reshape(-1).contiguous())
        if spec is None:
            tk = clm_gpu.sample_or_argmax(lg)
            return as_bits(o), lg.cpu().numpy(), tk.cpu().numpy()
        dp, dtok, ua, ur = (to_torch(spec[k][np.asarray(sel)]) for k in ("draft_probs", "draft_tokens",
                                                                          "u_accept", "u_resample"))
        toks, num = clm_gpu.spec_verify(lg.view(len(sel), c.Kq, c.V), dp, dtok, ua, ur, c.temperature)
        return as_bits(o), lg.cpu().numpy(), (toks.cpu().numpy(), num.cpu().numpy())

    full = run(np.arange(c.B))
    sel = np.random.default_rng(77).permutation(c.B)[:sub]
    part = run(sel)
    np.testing.assert_array_equal(part[0], full[0][sel])
    rows = (sel[:, None] * c.Kq + np.arange(c.Kq)[None, :]).reshape(-1)
    np.testing.assert_array_equal(part[1].view(np.uint32), full[1][rows].view(np.uint32))
    if spec is None:
        np.testing.assert_array_equal(part[2], full[2][rows])
    else:
        np.testing.assert_array_equal(part[2][0], full[2][0][sel])
        np.testing.assert_array_equal(part[2][1], full[2][1][sel])
    print(f"compaction c{cfg}: {sub} of {c.B} streams bit-identical")


def test_checked_mode_reports_bad_device_data(clm_gpu):
    """With checked mode switched on in-process (clm_set_checked), every call
    validates its device-resident indices first: an out-of-range block id, a
    length beyond the block table, a head id, a uniform and a drafted token
    each give CLM_ERR_DEVICE_DATA and launch nothing; valid data passes and
    the results match the unchecked calls bit for bit."""
    import torch
    x = inputs(4)
    c = x.cfg
    d = Dev(x, include_new=False)
    prev = clm_gpu.set_checked(True)
    try:
        def status(fn):
            try:
                fn()
                return 0
            except clm_gpu.ClmError as e:
                return e.status

        bad_bt = d.block_table.clone()
        bad_bt[3, 0] = x.num_blocks + 5                   # block id past the pool
        k_before = as_bits(d.k_cache)
        assert status(lambda: clm_gpu.kv_cache_append(d.k_new, d.v_new, d.k_cache, d.v_cache, bad_bt,
                                                      d.len_before)) == -6
        assert np.array_equal(as_bits(d.k_cache), k_before)     # nothing launched
        bad_lb = d.len_before.clone()
        bad_lb[1] = x.max_blocks * c.block_size                 # no room for the new rows
        assert status(lambda: clm_gpu.kv_cache_append(d.k_new, d.v_new, d.k_cache, d.v_cache, d.block_table,
                                                      bad_lb)) == -6
        assert status(lambda: clm_gpu.kv_cache_append(d.k_new, d.v_new, d.k_cache, d.v_cache, d.block_table,
                                                      d.len_before)) == 0
        bad_len = d.kv_len.clone()
        bad_len[0] = d.max_kv_len + 1                           # above the caller's bound
        assert status(lambda: clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, d.block_table, bad_len,
                                                       d.max_kv_len)) == -6
        assert status(lambda: clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, bad_bt, d.kv_len,
                                                       d.max_kv_len)) == -6
        o_chk = clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, d.block_table, d.kv_len, d.max_kv_len)
        h = o_chk.view(c.M, c.d_model)
        W3 = torch.stack([d.W[0]] * 3)
        hid = torch.zeros(c.M, dtype=torch.int32, device=h.device)
        hid[5] = 3                                              # only heads 0..2 exist
        assert status(lambda: clm_gpu.codebook_head(h, W3, hid)) == -6
        lg_chk = clm_gpu.codebook_head(h, d.W)
        u = torch.full((c.M,), 0.5, device=h.device)
        u[7] = 1.0                                              # uniforms lie in [0, 1)
        temp = torch.full((c.M,), 0.7, device=h.device)
        assert status(lambda: clm_gpu.sample_or_argmax(lg_chk, temp, u)) == -6
        vv = torch.full((c.M,), c.V + 1, dtype=torch.int32, device=h.device)   # mask past V
        assert status(lambda: clm_gpu.sample_or_argmax(lg_chk, None, None, vv)) == -6
        s = x.spec_inputs()
        dp, dtok, ua, ur = _spec_inputs_torch(s)
        bad_tok = dtok.clone()
        bad_tok[2, 1] = c.V
        assert status(lambda: clm_gpu.spec_verify(lg_chk.view(c.B, c.Kq, c.V), dp, bad_tok, ua, ur, 0.7)) == -6
        toks_chk, num_chk = clm_gpu.spec_verify(lg_chk.view(c.B, c.Kq, c.V), dp, dtok, ua, ur, 0.7)
    finally:
        clm_gpu.set_checked(prev)
    o = clm_gpu.decode_attention(d.q, d.k_cache, d.v_cache, d.block_table, d.kv_len, d.max_kv_len)
    lg = clm_gpu.codebook_head(o.view(c.M, c.d_model), d.W)
    toks, num = clm_gpu.spec_verify(lg.view(c.B, c.Kq, c.V), dp, dtok, ua, ur, 0.7)
    assert np.array_equal(as_bits(o), as_bits(o_chk))
    assert torch.equal(lg, lg_chk) and torch.equal(toks, toks_chk) and torch.equal(num, num_chk)


def test_codebook_head_rows_independent_of_batch(clm_gpu):
    """A row's logits are the same bits whatever else is in the call: the
    head always sums two fp32 chains (even and odd 32-wide k blocks), so the
    tile plan - 4 or 8 waves, 32..128 rows and 32..128 codebook entries per
    workgroup, chosen from M, V and G - changes no result.  Rows are taken
    from a 256-row call into calls of 100, 37, 16 and 1 rows (one stage) and
    into grouped calls over 3 stages; all against the oracle too."""
    import torch
    rng = np.random.default_rng(4242)
    d, V = 2048, 4096
    h = synth.f32_to_bf16_bits(rng.standard_normal((256, d)).astype(np.float32))
    W = synth.f32_to_bf16_bits((rng.standard_normal((3, V, d)) * 0.02).astype(np.float32))
    ht, Wt = to_torch(h, bf16=True), to_torch(W, bf16=True)
    full = clm_gpu.codebook_head(ht, Wt[0:1]).cpu().numpy()
    ref = oracle.codebook_head(synth.bf16_bits_to_f32(h), synth.bf16_bits_to_f32(W[0:1]))
    check_close(full, ref, "head 256 rows")
    for m in (100, 37, 16, 1):
        sel = np.sort(rng.choice(256, size=m, replace=False))
        part = clm_gpu.codebook_head(ht[torch.from_numpy(sel).to(ht.device)].contiguous(), Wt[0:1]).cpu().numpy()
        np.testing.assert_array_equal(part.view(np.uint32), full[sel].view(np.uint32), err_msg=f"M={m}")
    # grouped: every row of stage g equals the same row in a one-stage call on W[g]
    hid = rng.integers(0, 3, size=256).astype(np.int32)
    grouped = clm_gpu.codebook_head(ht, Wt, to_torch(hid)).cpu().numpy()
    for g in range(3):
        rows = np.nonzero(hid == g)[0]
        one = clm_gpu.codebook_head(ht[torch.from_numpy(rows).to(ht.device)].contiguous(), Wt[g:g + 1]).cpu().numpy()
        np.testing.assert_array_equal(grouped[rows].view(np.uint32), one.view(np.uint32), err_msg=f"stage {g}")
    check_close(grouped, oracle.codebook_head(synth.bf16_bits_to_f32(h), synth.bf16_bits_to_f32(W), hid),
                "grouped head 256 rows")


@pytest.mark.parametrize("Kq", [1, 6])
def test_decode_attention_closed_forms(clm_gpu, Kq):
    """Results fixed by the definition alone, on both kernels and across
    split merges (the 3000- and 1000-key streams span several splits):
    - a stream whose keys are all equal attends uniformly: each query's output
      is the plain mean of the values it sees (causal: query j of a block
      averages exactly kv_len - (Kq-1-j) rows; the 17- and 2-key streams make
      one row more or less show);
    - a query equal to 30/sqrt(D) times one visible key (a score of about 30
      for that key against a spread of about 3 for the others) returns that
      key's value row;
    - scores with a spread of about 100 (q and K entries of N(0, 10)) against
      the oracle."""
    rng = np.random.default_rng(777 + Kq)
    Hq, Hk, D, bs = 16, 8, 128, 16
    G = Hq // Hk
    lens = [3000, 1000, 17, max(Kq, 2), 2500, 64]
    kv_len, bt, kc, vc, q, keys, vals = _random_pool_case(rng, lens, Kq, Hq, Hk, D, bs)
    B = len(lens)
    # streams 0-3: every key row equal (per KV head)
    for b in (0, 1, 2, 3):
        n = int(kv_len[b])
        row = synth.f32_to_bf16_bits(rng.standard_normal((Hk, D)).astype(np.float32))
        for pos in range(n):
            kc[bt[b, pos // bs], :, pos % bs, :] = row
    # stream 4: each query row is 30 x the key at position t (visible to every query of the block)
    t_dom = 1234
    qf = synth.bf16_bits_to_f32(q)
    kf = synth.bf16_bits_to_f32(kc)
    for j in range(Kq):
        for h in range(Hq):
            qf[4, j, h] = 30.0 * kf[bt[4, t_dom // bs], h // G, t_dom % bs] / np.sqrt(D)
    # stream 5: large scores
    qf[5] *= 10.0
    q = synth.f32_to_bf16_bits(qf)
    qf = synth.bf16_bits_to_f32(q)
    blk5 = bt[5, :(64 + bs - 1) // bs]
    kc[blk5] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(kc[blk5]) * 10.0)
    scale = 1.0 / math.sqrt(D)
    o = clm_gpu.decode_attention(to_torch(q, bf16=True), to_torch(kc, bf16=True), to_torch(vc, bf16=True),
                                 to_torch(bt), to_torch(kv_len), int(kv_len.max()), scale=scale)
    of = bf16_tensor_to_f32(o)
    vf = synth.bf16_bits_to_f32(vc)
    for b in (0, 1, 2, 3):
        for j in range(Kq):
            n_j = int(kv_len[b]) - (Kq - 1 - j)
            pos = np.arange(n_j)
            mean = vf[bt[b, pos // bs], :, :, pos % bs].astype(np.float64).mean(axis=0)    # [Hk, D]
            want = np.repeat(mean, G, axis=0)                                               # [Hq, D]
            # exact up to fp32 sums and the bf16 output rounding
            check_close(of[b, j], want, f"equal keys: stream {b} query {j} averages its {n_j} rows",
                        atol=2e-3, rtol=8e-3)
    v_dom = vf[bt[4, t_dom // bs], :, :, t_dom % bs]                                        # [Hk, D]
    for j in range(Kq):
        check_close(of[4, j], np.repeat(v_dom, G, axis=0), f"dominant key: query {j}")
    keys5 = [synth.bf16_bits_to_f32(kc)[bt[5, np.arange(64) // bs], :, np.arange(64) % bs, :]]
    vals5 = [vf[bt[5, np.arange(64) // bs], :, :, np.arange(64) % bs]]
    ref5 = oracle.decode_attention(qf[5:6], keys5, vals5, kv_len[5:6], scale, Hk)
    check_close(of[5:6], ref5, "scores of magnitude ~100")


def test_binding_rejects_short_per_row_arrays(clm_gpu):
    """The binding refuses per-stream and per-row arrays shorter than the
    batch before any launch (a kernel would read past their ends)."""
    import torch
    dev = torch.device("cuda")
    B, Kq, Hq, Hk, D, bs, nb, V = 4, 2, 16, 8, 128, 16, 8, 64
    q = torch.zeros((B, Kq, Hq, D), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((nb, Hk, bs, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros((nb, Hk, D, bs), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((B, 2), dtype=torch.int32, device=dev)
    kl = torch.full((B,), 4, dtype=torch.int32, device=dev)
    short = torch.zeros(B - 1, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        clm_gpu.decode_attention(q, kc, vc, bt, short, 16)
    with pytest.raises(ValueError):
        clm_gpu.decode_attention(q, kc, vc, bt[:B - 1], kl, 16)
    k8 = torch.zeros((nb, Hk, D // 8, bs, 8), dtype=torch.uint8, device=dev)
    v8 = torch.zeros((nb, Hk, D, bs), dtype=torch.uint8, device=dev)
    sc = torch.ones((nb, Hk, bs), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        clm_gpu.decode_attention_fp8(q, k8, v8, sc, sc, bt, short, 16)
    kn = torch.zeros((B, Kq, Hk, D), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        clm_gpu.kv_cache_append_fp8(kn, kn, k8, v8, sc, sc, bt, short)
    logits = torch.zeros((B, V), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        clm_gpu.sample_or_argmax(logits, torch.ones(B - 1, device=dev), torch.ones(B - 1, device=dev))
    with pytest.raises(ValueError):
        clm_gpu.sample_or_argmax(logits, vocab_valid=short)
    tl = torch.zeros((B, Kq, V), dtype=torch.float32, device=dev)
    dt = torch.zeros((B, Kq), dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        clm_gpu.spec_verify(tl, tl, dt, torch.zeros((B, Kq - 1), device=dev), torch.zeros(B, device=dev), 0.7)
    with pytest.raises(ValueError):
        clm_gpu.spec_verify(tl, tl, dt, torch.zeros((B, Kq), device=dev), torch.zeros(B - 1, device=dev), 0.7)
    h = torch.zeros((B, Hq * D), dtype=torch.bfloat16, device=dev)
    W = torch.zeros((2, V, Hq * D), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        clm_gpu.codebook_head(h, W, short)
