"""Host-side checks of libclm.so that need no GPU: it loads, exports every
function include/clm.h declares, and rejects bad arguments before any HIP call
(so these calls never touch a device)."""

import ctypes as C
import os
import re

import pytest

import codec_language_model_amd as clm
from codec_language_model_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "clm.h")

INVALID, UNSUPPORTED, CAPACITY, WORKSPACE = -1, -2, -3, -4
P = C.c_void_p(0x100000)          # a non-null, 256-byte aligned stand-in; never dereferenced
N = C.c_void_p(0)
S = C.c_void_p(0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(clm_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return clm.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"binding lacks {n}"
    assert set(_lib.SIGNATURES) == set(names)


def test_checked_mode_switch(lib):
    prev = lib.clm_set_checked(1)
    try:
        assert lib.clm_set_checked(1) == 1
        assert lib.clm_set_checked(0) == 1
        assert lib.clm_set_checked(0) == 0
        # host validation still runs first: no HIP call for a bad argument
        lib.clm_set_checked(1)
        assert append(lib, B=0) == INVALID
        assert attn(lib, q=N) == INVALID
    finally:
        lib.clm_set_checked(prev)
    # the binding's wrapper returns the previous setting as a bool
    assert clm.set_checked(True) is bool(prev)
    assert clm.set_checked(bool(prev)) is True


def test_status_strings_and_version(lib):
    for code, name in _lib.STATUS.items():
        assert lib.clm_status_string(code).decode() == name
    assert lib.clm_status_string(42).decode() == "CLM_ERR_UNKNOWN"
    assert lib.clm_version() >= 100


def test_missing_library_fails_loudly(tmp_path):
    saved = _lib._lib
    _lib._lib = None
    try:
        with pytest.raises(RuntimeError, match="no CPU fallback"):
            _lib.load(str(tmp_path / "libclm.so"))
    finally:
        _lib._lib = saved


def append(lib, **kw):
    a = dict(k_new=P, v_new=P, k_cache=P, v_cache=P, bt=P, max_blocks=8, lb=P, B=2, T=1, H=8, D=128,
             bs=16, nb=100, dt=1)
    a.update(kw)
    return lib.clm_kv_cache_append(a["k_new"], a["v_new"], a["k_cache"], a["v_cache"], a["bt"],
                                   a["max_blocks"], a["lb"], a["B"], a["T"], a["H"], a["D"], a["bs"],
                                   a["nb"], a["dt"], S)


def test_append_argument_errors(lib):
    assert append(lib, k_new=N) == INVALID
    assert append(lib, B=0) == INVALID
    assert append(lib, T=0) == INVALID
    assert append(lib, k_cache=C.c_void_p(0x100008)) == INVALID     # not 16-byte aligned
    assert append(lib, D=96) == UNSUPPORTED
    assert append(lib, bs=24) == UNSUPPORTED
    assert append(lib, bs=512) == UNSUPPORTED
    assert append(lib, dt=7) == UNSUPPORTED
    assert append(lib, T=129, max_blocks=8, bs=16) == CAPACITY


def attn(lib, ws_bytes=None, **kw):
    a = dict(q=P, k=P, v=P, bt=P, max_blocks=64, kv_len=P, max_kv_len=1000, o=P, B=4, Kq=1, Hq=16, Hk=8,
             D=128, bs=16, nb=300, scale=0.088, dt=1, ws=P)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.clm_decode_attention_workspace_size(a["B"], a["Kq"], a["Hq"], a["Hk"], a["D"],
                                                           a["max_kv_len"]) - 1
    return lib.clm_decode_attention(a["q"], a["k"], a["v"], a["bt"], a["max_blocks"], a["kv_len"],
                                    a["max_kv_len"], a["o"], a["B"], a["Kq"], a["Hq"], a["Hk"], a["D"],
                                    a["bs"], a["nb"], C.c_float(a["scale"]), a["dt"], a["ws"], ws_bytes, S)


def test_attention_argument_errors(lib):
    assert attn(lib, q=N) == INVALID
    assert attn(lib, Hq=12, Hk=8) == INVALID
    assert attn(lib, max_kv_len=0) == INVALID
    assert attn(lib, Kq=6, max_kv_len=5) == INVALID
    assert attn(lib, scale=float("inf")) == INVALID
    assert attn(lib, D=80) == UNSUPPORTED
    assert attn(lib, Hq=34, Hk=2) == UNSUPPORTED          # 17 query heads per KV head
    assert attn(lib, Kq=6, Hq=32, Hk=8) == UNSUPPORTED    # 4 * 6 = 24 rows per KV head
    assert attn(lib, B=5000) == UNSUPPORTED
    assert attn(lib, B=4096, Hq=32, Hk=32, ws_bytes=1 << 40) == UNSUPPORTED   # 131072 (stream, KV head) pairs
    assert attn(lib) == WORKSPACE                          # one byte short
    assert attn(lib, ws=N, ws_bytes=1 << 30) == WORKSPACE
    assert attn(lib, ws=C.c_void_p(0x100010), ws_bytes=1 << 30) == WORKSPACE  # misaligned


def test_noalloc_attention_rejects_plans_beyond_its_scratch(lib):
    """The allocation-free attention takes plans up to 32 MiB of split
    partials; beyond that it returns WORKSPACE before any HIP call (here
    there is no GPU, so a HIP call would have given CLM_ERR_HIP)."""
    f = lib.clm_decode_attention_noalloc
    ws = lib.clm_decode_attention_workspace_size
    def call(B, max_kv_len, **kw):
        a = dict(q=P, Hq=16, Hk=8, D=128, Kq=1)
        a.update(kw)
        return f(a["q"], P, P, P, 4096, P, max_kv_len, P, B, a["Kq"], a["Hq"], a["Hk"], a["D"], 16, 1 << 20,
                 C.c_float(0.088), 1, S)
    assert ws(256, 1, 16, 8, 128, 65536) > 32 << 20
    assert call(256, 65536) == WORKSPACE
    assert ws(4096, 1, 16, 8, 128, 4096) > 32 << 20
    assert call(4096, 4096) == WORKSPACE
    assert call(256, 8192, q=N) == INVALID                 # argument errors come first
    assert call(256, 8192, Hq=12) == INVALID
    assert call(256, 8192, D=96) == UNSUPPORTED


def test_workspace_size_query(lib):
    f = lib.clm_decode_attention_workspace_size
    assert f(0, 1, 16, 8, 128, 100) == 0
    assert f(4, 1, 16, 8, 96, 100) == 0
    assert f(4, 6, 16, 8, 128, 5) == 0
    small = f(16, 1, 16, 8, 128, 1500)
    big = f(256, 1, 16, 8, 128, 8192)
    assert 0 < small < big
    # (m, l) + accumulators for every (stream, KV head, split, row): at 256
    # streams of up to 8192 keys a split is 1024 tokens, so 8 splits
    assert big >= 256 * 8 * 8 * 2 * 130 * 4
    # more than 65536 (stream, KV head) pairs, with a valid head grouping
    assert f(4096, 1, 32, 32, 128, 100) == 0
    assert f(2048, 1, 32, 32, 128, 100) > 0             # exactly 65536 pairs
    assert f(4096, 1, 16, 32, 128, 100) == 0            # H_q not a multiple of H_kv


def _attn_ws(B, Hk, max_splits, nr_tmpl, D):
    """Bytes of the split partials: (m, l) and D accumulators per (stream, KV
    head, split, row), each array rounded up to 256 bytes."""
    slots = B * Hk * max_splits * nr_tmpl
    up = lambda x: (x + 255) // 256 * 256
    return up(slots * 2 * 4) + up(slots * D * 4)


def test_split_plan_rules(lib):
    """The split length, read back through the workspace size.  1-2 query rows
    per KV head: the largest power of two <= est / 512 in [64, 1024], with
    est = B * H_kv * max_kv_len / 2.  3-16 rows: the smallest of 64, 128,
    192, 256, 384, 512 at or above est / 768."""
    f = lib.clm_decode_attention_workspace_size
    # 256 x 1 query, max 8192: est 8.4 M -> 1024 tokens, 8 splits
    assert f(256, 1, 16, 8, 128, 8192) == _attn_ws(256, 8, 8, 2, 128)
    # 16 x 1 query, max 1500: est 96,000 -> 128 tokens, 12 splits
    assert f(16, 1, 16, 8, 128, 1500) == _attn_ws(16, 8, 12, 2, 128)
    # 32 x 6 queries (12 rows), max 1965: est 251,520 -> want 327.5 -> 384, 6 splits
    assert f(32, 6, 16, 8, 128, 1965) == _attn_ws(32, 8, 6, 12, 128)
    # 26 and 37 streams keep 384 tokens; 25 and 38 do not
    assert f(26, 6, 16, 8, 128, 1965) == _attn_ws(26, 8, 6, 12, 128)
    assert f(37, 6, 16, 8, 128, 1965) == _attn_ws(37, 8, 6, 12, 128)
    assert f(25, 6, 16, 8, 128, 1965) == _attn_ws(25, 8, 8, 12, 128)       # 256 tokens
    assert f(38, 6, 16, 8, 128, 1965) == _attn_ws(38, 8, 4, 12, 128)       # 512 tokens
    # 16 x 6 queries, max 2000: want 166.7 -> 192 tokens, 11 splits
    assert f(16, 6, 16, 8, 128, 2000) == _attn_ws(16, 8, 11, 12, 128)
    # long streams: 2 streams x 8 KV heads, max 100,000 keys: est 800,000 ->
    # 1024 tokens, 98 splits; one such stream alone: est 400,000 -> 512, 196
    assert f(2, 1, 16, 8, 128, 100000) == _attn_ws(2, 8, 98, 2, 128)
    assert f(1, 1, 16, 8, 128, 100000) == _attn_ws(1, 8, 196, 2, 128)


def test_head_workspace_size_queries(lib):
    """Every tile plan of the workloads' shapes runs without scratch (the
    workspace argument is accepted and may be NULL); invalid sizes give 0."""
    f = lib.clm_codebook_head_workspace_size
    for M, d, V, G in [(1, 256, 4096, 1), (16, 2048, 16384, 1), (64, 2048, 4096, 3), (192, 2048, 4096, 1),
                       (256, 2048, 16384, 1), (65536, 2048, 4096, 8)]:
        assert f(M, d, V, G, 1) == 0
        assert f(M, d, V, G, 0) == 0
    assert f(0, 2048, 4096, 1, 1) == 0 and f(70000, 2048, 4096, 1, 1) == 0 and f(4, 2048, 4096, 9, 1) == 0
    g = lib.clm_codebook_head_mlp_workspace_size
    assert g(256, 2048, 4096, 16384, 1) == 0 and g(64, 2048, 4096, 4096, 3) == 0


def test_two_layer_head_argument_errors(lib):
    W = (C.c_void_p * 2)(0x100000, 0x200000)
    f = lib.clm_codebook_head_mlp
    assert f(P, W, W, 2, N, P, P, 16, 2048, 4096, 4096, 1, N, 0, S) == INVALID      # G > 1 needs head_id
    assert f(P, W, W, 1, N, N, P, 16, 2048, 4096, 4096, 1, N, 0, S) == INVALID      # act missing
    assert f(P, W, W, 1, N, P, P, 16, 2048, 4000, 4096, 1, N, 0, S) == UNSUPPORTED  # F % 128
    assert f(P, W, W, 1, N, P, P, 16, 2000, 4096, 4096, 1, N, 0, S) == UNSUPPORTED  # d % 128
    assert f(P, W, W, 1, N, P, P, 16, 2048, 4096, 4096, 0, N, 0, S) == UNSUPPORTED  # fp32 not supported
    # a workspace, when given, must be 256-byte aligned
    assert f(P, W, W, 1, N, P, P, 16, 2048, 4096, 4096, 1, C.c_void_p(0x100040), 1 << 20, S) == WORKSPACE


def test_rope_append_argument_errors(lib):
    f = lib.clm_rope_kv_cache_append
    args = [P, P, P, P, P, P, 8, P, P, C.c_float(1e6), 4, 1, 16, 8, 128, 16, 64, 1, S]
    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a0=N) == INVALID                       # q missing
    assert call(a8=N) == INVALID                       # positions missing
    assert call(a9=C.c_float(1.0)) == INVALID          # base <= 1
    assert call(a9=C.c_float(float("nan"))) == INVALID
    assert call(a12=12) == INVALID                     # H_q % H_kv
    assert call(a14=96) == UNSUPPORTED                 # D
    assert call(a15=24) == UNSUPPORTED                 # block size
    assert call(a11=1000) == CAPACITY                  # T_new > max_blocks * bs


def test_rope_fp8_append_argument_errors(lib):
    f = lib.clm_rope_kv_cache_append_fp8
    args = [P, P, P, P, P, P, P, P, 8, P, P, C.c_float(1e6), 4, 1, 16, 8, 128, 16, 64, S]
    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a0=N) == INVALID                       # q missing
    assert call(a5=N) == INVALID                       # a scale array missing
    assert call(a10=N) == INVALID                      # positions missing
    assert call(a11=C.c_float(0.5)) == INVALID         # base <= 1
    assert call(a11=C.c_float(float("inf"))) == INVALID
    assert call(a14=12) == INVALID                     # H_q % H_kv
    assert call(a0=C.c_void_p(0x100008)) == INVALID    # q not 16-byte aligned
    assert call(a16=96) == UNSUPPORTED                 # D
    assert call(a17=24) == UNSUPPORTED                 # block size
    assert call(a13=1000) == CAPACITY                  # T_new > max_blocks * bs


def test_head_sampler_verify_argument_errors(lib):
    Ws = (C.c_void_p * 3)(0x100000, 0x200000, 0x300000)
    head = lib.clm_codebook_head
    assert head(P, Ws, 3, N, P, 64, 2048, 4096, 1, N, 0, S) == INVALID   # G > 1 needs head_id
    assert head(P, Ws, 9, P, P, 64, 2048, 4096, 1, N, 0, S) == INVALID
    assert head(P, Ws, 1, N, P, 0, 2048, 4096, 1, N, 0, S) == INVALID
    assert head(P, Ws, 1, N, P, 4, 2000, 4096, 1, N, 0, S) == UNSUPPORTED
    assert head(N, Ws, 1, N, P, 4, 2048, 4096, 1, N, 0, S) == INVALID
    assert head(P, Ws, 1, N, P, 70000, 2048, 4096, 1, N, 0, S) == UNSUPPORTED
    assert head(P, Ws, 1, N, P, 64, 2048, 4096, 1, C.c_void_p(0x100010), 4096, S) == WORKSPACE  # misaligned
    assert lib.clm_sample_or_argmax(P, 4, 100, 99, N, N, N, P, S) == INVALID       # ld < V
    assert lib.clm_sample_or_argmax(P, 4, 100, 100, P, N, N, P, S) == INVALID      # T without u
    assert lib.clm_sample_or_argmax(P, 4, (1 << 20) + 1, (1 << 20) + 1, N, N, N, P, S) == UNSUPPORTED
    assert lib.clm_spec_verify(P, P, P, P, P, C.c_float(-0.1), 4, 6, 4096, P, P, S) == INVALID
    assert lib.clm_spec_verify(P, P, P, P, P, C.c_float(float("nan")), 4, 6, 4096, P, P, S) == INVALID
    assert lib.clm_spec_verify(P, P, P, P, P, C.c_float(0.7), 4, 17, 4096, P, P, S) == UNSUPPORTED
    assert lib.clm_spec_verify(P, N, P, P, P, C.c_float(0.7), 4, 6, 4096, P, P, S) == INVALID


def test_oracle_bf16_rounding_pins():
    import numpy as np
    import oracle
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.5, 0.0, 65504.0],
                 np.float32)
    want = np.array([1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -2.5, 0.0, 65536.0], np.float32)
    np.testing.assert_array_equal(oracle.round_to_bf16(x), want)
    import torch
    y = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 100
    np.testing.assert_array_equal(oracle.round_to_bf16(y),
                                  torch.from_numpy(y).to(torch.bfloat16).to(torch.float32).numpy())


def test_decode_loop_host_checks(lib):
    """The loop's host-side checks need no GPU: bucket choice, and argument
    errors of create / launch / destroy / advance before any HIP call."""
    import ctypes as C
    from codec_language_model_amd._lib import DecodeStepDesc
    sizes = (C.c_int32 * 3)(16, 64, 256)
    pick = lib.clm_pick_bucket
    ptr = C.cast(sizes, C.c_void_p)
    assert [pick(ptr, 3, B) for B in (1, 16, 17, 64, 65, 256, 257)] == [0, 0, 1, 1, 2, 2, -1]
    unsorted = (C.c_int32 * 3)(256, 16, 64)
    assert pick(C.cast(unsorted, C.c_void_p), 3, 20) == 2
    assert pick(N, 3, 5) == -1 and pick(ptr, 0, 5) == -1
    h = C.c_void_p()
    d = DecodeStepDesc(B=4, Kq=1, H_q=16, H_kv=8, D=128, block_size=16, num_blocks=64, max_blocks=8,
                       max_kv_len=128, G=1, V=4096, dt=1, k_cache=0x100000, v_cache=0x100000,
                       block_table=0x100000, len_before=0x100000, kv_len=0x100000, k_new=0x100000,
                       v_new=0x100000, q=0x100000, W=0x100000, o=0x100000, logits=0x100000, tokens=0x100000,
                       mode=0)
    create = lib.clm_decode_loop_create
    assert create(None, 4, C.byref(h)) == INVALID
    assert create(C.byref(d), 0, C.byref(h)) == INVALID
    assert create(C.byref(d), 1025, C.byref(h)) == INVALID
    d.tokens = 0
    assert create(C.byref(d), 4, C.byref(h)) == INVALID          # greedy needs tokens
    d.tokens, d.mode = 0x100000, 1
    assert create(C.byref(d), 4, C.byref(h)) == INVALID          # sampling needs temperature, uniforms
    d.mode = 2
    assert create(C.byref(d), 4, C.byref(h)) == INVALID          # verification needs the draft arrays
    d.mode = 3
    assert create(C.byref(d), 4, C.byref(h)) == INVALID          # bonus verification: the draft arrays ...
    d.draft_probs = d.draft_tokens = d.u_accept = d.u_resample = d.out_tokens = d.num_emitted = 0x100000
    assert create(C.byref(d), 4, C.byref(h)) == INVALID          # ... and Kq >= 2 (last token + a draft)
    d.draft_probs = d.draft_tokens = d.u_accept = d.u_resample = d.out_tokens = d.num_emitted = 0
    d.mode = 7
    assert create(C.byref(d), 4, C.byref(h)) == INVALID
    d.mode = 0
    d.k_scale = 0x100000                                         # FP8 cache: both scale arrays ...
    assert create(C.byref(d), 4, C.byref(h)) == INVALID
    d.v_scale = 0x100000
    assert create(C.byref(d), 4, C.byref(h)) == UNSUPPORTED      # ... and a caller workspace
    d.attn_workspace, d.attn_workspace_bytes = 0x100000, 1 << 20
    d.dt = 0
    assert create(C.byref(d), 4, C.byref(h)) == UNSUPPORTED      # bf16 queries only
    d.dt, d.k_scale, d.v_scale, d.attn_workspace, d.attn_workspace_bytes = 1, 0, 0, 0, 0
    d.W2, d.F = 0x100000, 4096                                   # two-layer head: the activation scratch ...
    assert create(C.byref(d), 4, C.byref(h)) == INVALID
    d.act, d.dt = 0x100000, 0
    assert create(C.byref(d), 4, C.byref(h)) == UNSUPPORTED      # ... and bf16
    d.W2, d.F, d.act, d.dt = 0, 0, 0, 1
    prev = lib.clm_set_checked(1)
    try:
        assert create(C.byref(d), 4, C.byref(h)) == UNSUPPORTED  # checked mode synchronises
    finally:
        lib.clm_set_checked(prev)
    assert lib.clm_decode_loop_launch(N, S) == INVALID
    assert lib.clm_decode_loop_destroy(N) == INVALID
    assert lib.clm_advance_lengths(N, P, N, N, 4, 1, S) == INVALID
    assert lib.clm_advance_lengths(P, P, N, N, 0, 1, S) == INVALID
    assert lib.clm_advance_lengths(P, P, N, N, 4, 0, S) == INVALID


def test_host_validation_under_sanitizers(tmp_path):
    """The host code of the library (argument validation, launch planning,
    checked-mode plumbing, the decode-loop builder) built for the CPU alone
    with AddressSanitizer and UndefinedBehaviorSanitizer, kernel launches
    replaced by stubs that report no device, and driven through every entry
    point with good and bad arguments (tests/host_sanitize/main.cpp).  Any
    sanitizer finding aborts the run; every status must be the documented one."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("needs g++ and the ROCm headers")
    csrc = os.path.join(ROOT, "codec_language_model_amd", "csrc")
    here = os.path.join(ROOT, "tests", "host_sanitize")
    exe = str(tmp_path / "clm_host_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"),
           os.path.join(csrc, "abi.cpp"), os.path.join(csrc, "loop.cpp"), os.path.join(csrc, "plan.cpp"),
           os.path.join(here, "stubs.cpp"), os.path.join(here, "main.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "ok: 0 mismatches" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
