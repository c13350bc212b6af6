"""clm_decode_attention_noalloc: the allocation-free form of decode attention
(split partials in the library's static per-GPU scratch) against the
workspace form, bit for bit, on consecutive calls of decreasing size through
the C ABI."""

import ctypes as C
import math
import sys

import numpy as np
import pytest

import synth
from parity import to_torch

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy().view(np.uint32)


def test_noalloc_attention_matches_workspace_attention(clm_gpu):
    import torch
    lib = clm_gpu.load()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    # 256 streams (the benchmark's launch), then 32 x 6-query blocks, then 16
    # streams and the one-stream fp32 step: each call smaller than the last
    for cfg, B in [(5, None), (4, None), (2, None), (1, None)]:
        print(f"\n[gpu-case] noalloc workload {cfg}", file=sys.stderr, flush=True)
        x = synth.make_inputs(cfg, B=B)
        c = x.cfg
        bf = c.dtype == "bf16"
        kp, vp = x.build_pool(include_new=True)
        kc, vc = to_torch(kp, bf16=bf), to_torch(vp, bf16=bf)
        q = to_torch(x.q, bf16=bf)
        bt, kvl = to_torch(x.block_table), to_torch(x.kv_len)
        max_kv = int(x.kv_len.max())
        scale = 1.0 / math.sqrt(c.D)
        assert clm_gpu.decode_attention_workspace_size(c.B, c.Kq, c.H_q, c.H_kv, c.D, max_kv) <= 32 << 20
        ref = clm_gpu.decode_attention(q, kc, vc, bt, kvl, max_kv, scale=scale)
        o = torch.full_like(q, float("nan"))
        st = lib.clm_decode_attention_noalloc(
            C.c_void_p(q.data_ptr()), C.c_void_p(kc.data_ptr()), C.c_void_p(vc.data_ptr()),
            C.c_void_p(bt.data_ptr()), bt.shape[1], C.c_void_p(kvl.data_ptr()), max_kv,
            C.c_void_p(o.data_ptr()), c.B, c.Kq, c.H_q, c.H_kv, c.D, c.block_size, kp.shape[0],
            C.c_float(scale), 1 if bf else 0, stream)
        assert st == 0, lib.clm_status_string(st)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(o), _bits(ref), err_msg=f"workload {cfg}")
        # the binding's wrapper of the same entry point
        o2 = torch.empty_like(q)
        clm_gpu.decode_attention_noalloc(q, kc, vc, bt, kvl, max_kv, scale=scale, out=o2)
        np.testing.assert_array_equal(_bits(o2), _bits(ref), err_msg=f"workload {cfg} (binding)")
        print(f"noalloc workload {cfg}: {c.B} streams bit-identical to the workspace call")
