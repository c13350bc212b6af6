"""GPU parity of the FP8 (E4M3) KV cache: the quantizing append bit-exact
against the oracle's quantizer, and attention over the FP8 cache against the
oracle's attention on the dequantized rows.  Empty slots hold NaN codes and
NaN scales, so any read of them shows."""

import math
import sys

import numpy as np
import pytest

import oracle
import synth
from oracle import fp8
from parity import bf16_tensor_to_f32, check_close, to_torch

pytestmark = pytest.mark.gpu

SMALL_B = {2: None, 3: 16, 4: None, 5: 24}


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield


def fp8_pool(x, include_new):
    """The bf16 synthetic pool quantized row by row (oracle quantizer), keys in
    the grouped layout [nb, H, D/8, bs, 8]; empty slots become NaN codes with
    NaN scales."""
    kp, vp = x.build_pool(include_new=include_new)
    kf = synth.bf16_bits_to_f32(kp)                               # [nb, H, bs, D]
    vf = synth.bf16_bits_to_f32(vp).transpose(0, 1, 3, 2)         # [nb, H, bs, D]
    out = []
    for rows in (kf, vf):
        empty = np.isnan(rows).any(axis=-1)
        codes, scale = fp8.quantize_rows(np.where(empty[..., None], 0.0, rows).astype(np.float32))
        codes[empty] = 0x7F
        scale = scale.astype(np.float32)
        scale[empty] = np.nan
        out.append((codes, scale))
    (kc, ks), (vc, vs) = out
    nb, H, bs, D = kc.shape
    kc = np.ascontiguousarray(kc.reshape(nb, H, bs, D // 8, 8).transpose(0, 1, 3, 2, 4))   # [nb, H, D/8, bs, 8]
    return kc, np.ascontiguousarray(vc.transpose(0, 1, 3, 2)), ks, vs


def dev(a):
    return to_torch(np.ascontiguousarray(a))


@pytest.mark.parametrize("cfg", [2, 4, 5])
def test_fp8_append_bit_exact(clm_gpu, cfg):
    import torch
    x = synth.make_inputs(cfg, B=SMALL_B[cfg])
    c = x.cfg
    kc, vc, ks, vs = fp8_pool(x, include_new=False)
    dk, dv, dks, dvs = dev(kc), dev(vc), dev(ks), dev(vs)
    clm_gpu.kv_cache_append_fp8(to_torch(x.k_new, bf16=True), to_torch(x.v_new, bf16=True), dk, dv, dks, dvs,
                                dev(x.block_table), dev(x.len_before), block_size=c.block_size)
    rk, rv, rks, rvs = fp8.fp8_kv_cache_append(kc, vc, ks, vs, x.block_table, x.len_before,
                                               synth.bf16_bits_to_f32(x.k_new), synth.bf16_bits_to_f32(x.v_new),
                                               c.block_size)
    np.testing.assert_array_equal(dk.cpu().numpy(), rk)
    np.testing.assert_array_equal(dv.cpu().numpy(), rv)
    np.testing.assert_array_equal(dks.cpu().numpy().view(np.uint32), rks.view(np.uint32))
    np.testing.assert_array_equal(dvs.cpu().numpy().view(np.uint32), rvs.view(np.uint32))
    del torch


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_fp8_attention_parity(clm_gpu, cfg):
    x = synth.make_inputs(cfg, B=SMALL_B[cfg])
    c = x.cfg
    kc, vc, ks, vs = fp8_pool(x, include_new=True)
    scale = 1.0 / math.sqrt(c.D)
    o = clm_gpu.decode_attention_fp8(to_torch(x.q, bf16=True), dev(kc), dev(vc), dev(ks), dev(vs),
                                     dev(x.block_table), dev(x.kv_len), int(x.kv_len.max()), scale=scale)
    keys, vals = [], []
    for b in range(c.B):
        K, V = fp8.gather_dequantized(kc, vc, ks, vs, x.block_table, b, int(x.kv_len[b]), c.block_size)
        keys.append(K)
        vals.append(V)
    ref = oracle.decode_attention(synth.bf16_bits_to_f32(x.q), keys, vals, x.kv_len, scale, c.H_kv)
    err = check_close(bf16_tensor_to_f32(o), ref, f"fp8 attention c{cfg}")
    print(f"fp8 attention c{cfg}: max abs err {err:.3g}")


def test_fp8_append_then_attention(clm_gpu):
    """The chained pair: quantizing append of the step's rows, then attention
    over the cache that now holds them."""
    x = synth.make_inputs(4)
    c = x.cfg
    kc, vc, ks, vs = fp8_pool(x, include_new=False)
    dk, dv, dks, dvs = dev(kc), dev(vc), dev(ks), dev(vs)
    bt, kl = dev(x.block_table), dev(x.kv_len)
    clm_gpu.kv_cache_append_fp8(to_torch(x.k_new, bf16=True), to_torch(x.v_new, bf16=True), dk, dv, dks, dvs,
                                bt, dev(x.len_before), block_size=c.block_size)
    scale = 1.0 / math.sqrt(c.D)
    o = clm_gpu.decode_attention_fp8(to_torch(x.q, bf16=True), dk, dv, dks, dvs, bt, kl, int(x.kv_len.max()),
                                     scale=scale)
    rk, rv, rks, rvs = fp8.fp8_kv_cache_append(kc, vc, ks, vs, x.block_table, x.len_before,
                                               synth.bf16_bits_to_f32(x.k_new), synth.bf16_bits_to_f32(x.v_new),
                                               c.block_size)
    keys, vals = [], []
    for b in range(c.B):
        K, V = fp8.gather_dequantized(rk, rv, rks, rvs, x.block_table, b, int(x.kv_len[b]), c.block_size)
        keys.append(K)
        vals.append(V)
    ref = oracle.decode_attention(synth.bf16_bits_to_f32(x.q), keys, vals, x.kv_len, scale, c.H_kv)
    check_close(bf16_tensor_to_f32(o), ref, "fp8 append + attention c4")



def test_fp8_attention_many_streams(clm_gpu):
    """More than 512 streams: the register-staged kernel (the LDS-staged one
    takes up to 512).  520 streams of 1..64 keys over random E4M3 codes (no
    NaN codes) and scales in [0.002, 0.01]; every 13th stream is checked
    against the oracle on the dequantized rows."""
    rng = np.random.default_rng(520)
    B, Hq, Hk, D, bs = 520, 16, 8, 128, 16
    kv_len = rng.integers(1, 65, size=B).astype(np.int32)
    pages = (kv_len + bs - 1) // bs
    nb = int(pages.sum()) + 2
    perm = rng.permutation(nb).astype(np.int32)
    max_blocks = int(pages.max())
    bt = np.zeros((B, max_blocks), np.int32)
    o_ = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[o_:o_ + pages[b]]
        o_ += pages[b]
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    kc = finite[rng.integers(0, finite.size, size=(nb, Hk, D // 8, bs, 8))]
    vc = finite[rng.integers(0, finite.size, size=(nb, Hk, D, bs))]
    ks = rng.uniform(0.002, 0.01, size=(nb, Hk, bs)).astype(np.float32)
    vs = rng.uniform(0.002, 0.01, size=(nb, Hk, bs)).astype(np.float32)
    q_bits = synth.f32_to_bf16_bits(rng.standard_normal((B, 1, Hq, D)).astype(np.float32))
    scale = 1.0 / math.sqrt(D)
    o = clm_gpu.decode_attention_fp8(to_torch(q_bits, bf16=True), dev(kc), dev(vc), dev(ks), dev(vs),
                                     dev(bt), dev(kv_len), int(kv_len.max()), scale=scale)
    idx = np.arange(0, B, 13)
    keys, vals = [], []
    for b in idx:
        K, V = fp8.gather_dequantized(kc, vc, ks, vs, bt, int(b), int(kv_len[b]), bs)
        keys.append(K)
        vals.append(V)
    ref = oracle.decode_attention(synth.bf16_bits_to_f32(q_bits)[idx], keys, vals, kv_len[idx], scale, Hk)
    check_close(bf16_tensor_to_f32(o)[idx], ref, "fp8 attention, 520 streams (sampled)")



def _random_fp8_pool(rng, nb, Hk, D, bs):
    """Uniform E4M3 codes without the two NaN codes, and row scales in
    [0.002, 0.01] (max|x|/448 for rows of N(0,1) values is about 0.007)."""
    def codes(shape):
        c = rng.integers(0, 254, size=shape, dtype=np.uint8)
        return c + (c >= 0x7F).astype(np.uint8)
    return (codes((nb, Hk, D // 8, bs, 8)), codes((nb, Hk, D, bs)),
            rng.uniform(0.002, 0.01, size=(nb, Hk, bs)).astype(np.float32),
            rng.uniform(0.002, 0.01, size=(nb, Hk, bs)).astype(np.float32))


# the oracle's decoder applied once to every code: a lookup table of its values
_E4M3 = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))


def _stream_rows(kc, vc, ks, vs, block_table, b, n, bs):
    """Stream b's first n positions as dequantized K, V [n, H, D] float64:
    code value (the oracle's decoder) times the row's scale, as the oracle's
    dequantize_rows computes it."""
    pos = np.arange(n)
    blk = block_table[b, pos // bs]
    slot = pos % bs
    H = kc.shape[1]
    kr = kc[blk, :, :, slot, :].reshape(n, H, -1)                 # [n, H, D]
    vr = vc[blk, :, :, slot]                                      # [n, H, D]
    return (_E4M3[kr] * ks[blk, :, slot].astype(np.float64)[..., None],
            _E4M3[vr] * vs[blk, :, slot].astype(np.float64)[..., None])


def test_fp8_attention_full_size(clm_gpu):
    """The 256-stream launch that the FP8 benchmark times (log-uniform
    64..8192 keys, 1024-token splits, LDS-staged matrix-core kernel, merge
    pass) over random E4M3 codes and scales of the pool's shapes: every
    stream's output against the oracle on the dequantized rows."""
    x = synth.make_inputs(5)
    c = x.cfg
    rng = np.random.default_rng(256)
    kc, vc, ks, vs = _random_fp8_pool(rng, x.num_blocks, c.H_kv, c.D, c.block_size)
    scale = 1.0 / math.sqrt(c.D)
    o = clm_gpu.decode_attention_fp8(to_torch(x.q, bf16=True), dev(kc), dev(vc), dev(ks), dev(vs),
                                     dev(x.block_table), dev(x.kv_len), int(x.kv_len.max()), scale=scale)
    q = synth.bf16_bits_to_f32(x.q)
    ref = np.empty(q.shape, np.float64)
    for b in range(c.B):                 # one stream at a time keeps the host memory small
        K, V = _stream_rows(kc, vc, ks, vs, x.block_table, b, int(x.kv_len[b]), c.block_size)
        ref[b:b + 1] = oracle.decode_attention(q[b:b + 1], [K], [V], x.kv_len[b:b + 1], scale, c.H_kv)
    err = check_close(bf16_tensor_to_f32(o), ref, "fp8 attention, all 256 streams")
    print(f"fp8 attention full size: max abs err {err:.3g}")


@pytest.mark.parametrize("cfg,bs,D", [(2, 32, 128), (4, 64, 128), (2, 16, 64), (4, 32, 64)])
def test_fp8_block_sizes(clm_gpu, cfg, bs, D):
    """The FP8 append and attention with pages of 16 to 64 slots and head
    widths 128 and 64 (the block-size-generic kernels and the D = 64
    instantiations, LDS-staged attention)."""
    import dataclasses
    c = dataclasses.replace(synth.get_config(cfg), block_size=bs, D=D)
    x = synth.make_inputs(c)
    kc, vc, ks, vs = fp8_pool(x, include_new=False)
    dk, dv, dks, dvs = dev(kc), dev(vc), dev(ks), dev(vs)
    bt, kl = dev(x.block_table), dev(x.kv_len)
    clm_gpu.kv_cache_append_fp8(to_torch(x.k_new, bf16=True), to_torch(x.v_new, bf16=True), dk, dv, dks, dvs,
                                bt, dev(x.len_before), block_size=bs)
    rk, rv, rks, rvs = fp8.fp8_kv_cache_append(kc, vc, ks, vs, x.block_table, x.len_before,
                                               synth.bf16_bits_to_f32(x.k_new), synth.bf16_bits_to_f32(x.v_new), bs)
    np.testing.assert_array_equal(dk.cpu().numpy(), rk)
    np.testing.assert_array_equal(dv.cpu().numpy(), rv)
    scale = 1.0 / math.sqrt(c.D)
    o = clm_gpu.decode_attention_fp8(to_torch(x.q, bf16=True), dk, dv, dks, dvs, bt, kl, int(x.kv_len.max()),
                                     scale=scale)
    keys, vals = [], []
    for b in range(c.B):
        K, V = fp8.gather_dequantized(rk, rv, rks, rvs, x.block_table, b, int(x.kv_len[b]), bs)
        keys.append(K)
        vals.append(V)
    ref = oracle.decode_attention(synth.bf16_bits_to_f32(x.q), keys, vals, x.kv_len, scale, c.H_kv)
    check_close(bf16_tensor_to_f32(o), ref, f"fp8 attention c{cfg} block size {bs} D {D}")


@pytest.mark.parametrize("Kq", [1, 6])
def test_fp8_attention_split_boundaries(clm_gpu, Kq):
    """The FP8 kernel with lengths on and next to the 64-token split and the
    16-token tile boundaries (12 streams, a bound of 129 keys), one query and
    6-query blocks, random codes and scales, against the oracle on the
    dequantized rows."""
    rng = np.random.default_rng(640 + Kq)
    Hq, Hk, D, bs = 16, 8, 128, 16
    kv_len = np.array([max(Kq, 1), 15, 16, 17, 63, 64, 65, 127, 128, 129, 32, 48 if Kq == 1 else 70], np.int32)
    B = kv_len.size
    pages = (kv_len + bs - 1) // bs
    nb = int(pages.sum()) + 2
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.zeros((B, int(pages.max())), np.int32)
    o_ = 0
    for b in range(B):
        bt[b, :pages[b]] = perm[o_:o_ + pages[b]]
        o_ += pages[b]
    kc, vc, ks, vs = _random_fp8_pool(rng, nb, Hk, D, bs)
    q_bits = synth.f32_to_bf16_bits(rng.standard_normal((B, Kq, Hq, D)).astype(np.float32))
    scale = 1.0 / math.sqrt(D)
    o = clm_gpu.decode_attention_fp8(to_torch(q_bits, bf16=True), dev(kc), dev(vc), dev(ks), dev(vs), dev(bt),
                                     dev(kv_len), 129, scale=scale)
    keys, vals = [], []
    for b in range(B):
        K, V = _stream_rows(kc, vc, ks, vs, bt, b, int(kv_len[b]), bs)
        keys.append(K)
        vals.append(V)
    ref = oracle.decode_attention(synth.bf16_bits_to_f32(q_bits), keys, vals, kv_len, scale, Hk)
    check_close(bf16_tensor_to_f32(o), ref, f"fp8 attention at split boundaries, Kq={Kq}")


def test_fp8_append_special_rows(clm_gpu):
    """Rows the quantizer treats specially, bit-exact against the oracle's
    codes and scales: all +0 (scale 1), all -0 and mixed signed zeros (sign
    bits kept), a single nonzero entry, rows whose scale is 1 so small entries
    land on the subnormal codes, magnitudes near the ends of the bf16 range,
    and a row of bf16 subnormals (its scale is an fp32 subnormal)."""
    B, T, H, D, bs = 1, 10, 1, 128, 16
    rng = np.random.default_rng(8)
    rows = np.zeros((T, D), np.float32)
    rows[1] = -0.0
    rows[2, ::2] = -0.0
    rows[3, 17] = 1.0
    rows[4] = rng.uniform(-0.02, 0.02, D)
    rows[4, 5] = 448.0                                   # scale 1: the rest quantize on the subnormal steps
    rows[5] = rng.standard_normal(D) * 1e30
    rows[6] = rng.standard_normal(D) * 1e-30
    rows[7] = rng.standard_normal(D) * 2e-39             # bf16 subnormals
    rows[8] = rng.standard_normal(D)
    rows[8, 0] = -3.0e38                                 # near the largest bf16
    rows[9] = np.linspace(-448.0, 448.0, D)
    bits = synth.f32_to_bf16_bits(rows).reshape(B, T, H, D)
    vals = synth.bf16_bits_to_f32(bits)
    nb = 1
    bt = np.zeros((B, 1), np.int32)
    lb = np.zeros(B, np.int32)
    kc = np.zeros((nb, H, D // 8, bs, 8), np.uint8)
    vc = np.zeros((nb, H, D, bs), np.uint8)
    ks = np.zeros((nb, H, bs), np.float32)
    vs = np.zeros((nb, H, bs), np.float32)
    dk, dv, dks, dvs = dev(kc), dev(vc), dev(ks), dev(vs)
    clm_gpu.kv_cache_append_fp8(to_torch(bits, bf16=True), to_torch(bits, bf16=True), dk, dv, dks, dvs, dev(bt),
                                dev(lb), block_size=bs)
    rk, rv, rks, rvs = fp8.fp8_kv_cache_append(kc, vc, ks, vs, bt, lb, vals, vals, bs)
    for name, got, want in (("key codes", dk, rk), ("value codes", dv, rv)):
        np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=name)
    for name, got, want in (("key scales", dks, rks), ("value scales", dvs, rvs)):
        np.testing.assert_array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32), err_msg=name)


@pytest.mark.parametrize("cfg,offset,bs,D", [(4, 1000, 16, 128), (5, 123456, 16, 128), (4, 77, 32, 64)])
def test_fp8_rope_append(clm_gpu, cfg, offset, bs, D):
    """The rotary append into the FP8 cache at logical positions len_before +
    offset + t: the oracle rotates the new keys (fp64), then quantizes them
    from float32 with its quantizer.  The kernel rotates in fp32, so a key
    element whose scaled value sits at a rounding boundary may take the
    neighbouring code; everything else is exact:
    - key scales within 4 ulp, key codes equal except for at most 1 in 1000,
      each of those one step from the oracle's (or a zero of the other sign);
    - value codes and scales bit-exact (values are not rotated);
    - the rotated queries within the attention tolerance, as the bf16 rotary
      append is checked; every slot the append does not own unchanged.
    Head width 64 (32-slot pages) takes the kernel's other pairing: the two
    members of a rotation pair sit in lanes i and i + 32."""
    import dataclasses
    x = synth.make_inputs(dataclasses.replace(synth.get_config(cfg), block_size=bs, D=D), B=SMALL_B[cfg])
    c = x.cfg
    T = c.Kq
    kc, vc, ks, vs = fp8_pool(x, include_new=False)
    pos = (x.len_before[:, None] + offset + np.arange(T)[None, :]).astype(np.int32)
    q = to_torch(x.q, bf16=True)
    dk, dv, dks, dvs = dev(kc), dev(vc), dev(ks), dev(vs)
    clm_gpu.rope_kv_cache_append_fp8(q, to_torch(x.k_new, bf16=True), to_torch(x.v_new, bf16=True), dk, dv, dks,
                                     dvs, dev(x.block_table), dev(x.len_before), dev(pos), 1.0e6, block_size=bs)
    f32 = synth.bf16_bits_to_f32
    q_ref = oracle.rope(f32(x.q), pos[:, :, None], 1.0e6)
    k_rot = oracle.rope(f32(x.k_new), pos[:, :, None], 1.0e6).astype(np.float32)
    rk, rv, rks, rvs = fp8.fp8_kv_cache_append(kc, vc, ks, vs, x.block_table, x.len_before, k_rot,
                                               f32(x.v_new), bs)
    check_close(bf16_tensor_to_f32(q), q_ref, f"fp8 rope q c{cfg}")
    np.testing.assert_array_equal(dv.cpu().numpy(), rv, err_msg="value codes")
    np.testing.assert_array_equal(dvs.cpu().numpy().view(np.uint32), rvs.view(np.uint32), err_msg="value scales")
    gk, gks = dk.cpu().numpy(), dks.cpu().numpy()
    # scales: every slot; untouched ones are bit-equal, new ones within 4 ulp
    np.testing.assert_allclose(gks, rks, rtol=4 * 2.0 ** -23, atol=0)
    diff = gk != rk
    n_touched = c.B * T * c.H_kv * c.D
    assert diff.sum() <= max(1, n_touched // 1000), f"{diff.sum()} key codes differ of {n_touched}"
    g_mag, r_mag = gk[diff] & 0x7F, rk[diff] & 0x7F
    same_sign = (gk[diff] & 0x80) == (rk[diff] & 0x80)
    ok = (same_sign & (np.abs(g_mag.astype(int) - r_mag.astype(int)) == 1)) | ((g_mag == 0) & (r_mag == 0))
    assert ok.all(), list(zip(gk[diff][~ok][:8], rk[diff][~ok][:8]))
    # every differing code belongs to a slot this append wrote
    touched = np.zeros(gk.shape[:2] + gk.shape[3:4], bool)      # [nb, H, bs]
    for b in range(c.B):
        for t in range(T):
            p_ = int(x.len_before[b]) + t
            touched[int(x.block_table[b, p_ // bs]), :, p_ % bs] = True
    assert not (diff.any(axis=(2, 4)) & ~touched).any(), "a slot the append does not own changed"
    print(f"fp8 rope append c{cfg}: {int(diff.sum())} of {n_touched} key codes one step from the oracle's")
