"""codec_language_model_amd - one batched decode step of a codec-language-model
TTS generator on AMD Instinct MI355X (gfx950).

The computation lives in libclm.so (hand-written HIP kernels behind the C ABI
in include/clm.h).  This module only marshals torch tensors into that ABI:
it checks device, dtype, shape and contiguity, passes data pointers and torch's
current HIP stream, and raises ClmError on a non-zero status.  torch provides
device memory and streams; no step of the computation runs here.

Calls (names follow the C ABI):
  kv_cache_append, decode_attention, codebook_head, sample_or_argmax,
  spec_verify, decode_attention_workspace_size
"""

from __future__ import annotations

import ctypes as C
import functools
import math

from . import _lib
from ._lib import CLM_BF16, CLM_F32, STATUS

__all__ = [
    "ClmError", "load", "kv_cache_append", "rope_kv_cache_append", "kv_cache_append_fp8", "decode_attention",
    "decode_attention_fp8", "decode_attention_workspace_size", "decode_attention_noalloc",
    "codebook_head", "codebook_head_mlp", "codebook_head_workspace_size", "codebook_head_mlp_workspace_size",
    "sample_or_argmax", "spec_verify", "spec_verify_bonus",
    "rope_kv_cache_append_fp8", "Workspace", "set_checked", "advance_lengths", "DecodeLoop", "pick_bucket",
]


class ClmError(RuntimeError):
    def __init__(self, call: str, status: int):
        super().__init__(f"{call} returned {status} ({STATUS.get(status, 'unknown')})")
        self.status = status


def load():
    return _lib.load()


def set_checked(on: bool) -> bool:
    """Checked mode on or off (clm_set_checked); returns the previous setting.
    In checked mode every call first validates its device-resident indices
    and raises ClmError with CLM_ERR_DEVICE_DATA when one is out of range."""
    return bool(load().clm_set_checked(1 if on else 0))


def _torch():
    import torch
    return torch


def _check(call: str, status: int):
    if status != 0:
        raise ClmError(call, status)


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return CLM_BF16
    if t.dtype == torch.float32:
        return CLM_F32
    raise TypeError(f"unsupported element type {t.dtype} (bfloat16 or float32)")


def _cuda(name, t, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


def _out(name, t, shape, dtype):
    """A caller-supplied output: a contiguous GPU tensor of exactly this shape
    and element type (the kernels write every element of that shape)."""
    _cuda(name, t, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _rows(call, B, **arrays):
    """Per-stream device arrays must have B rows: a shorter one would be read
    past its end by the kernels."""
    for name, t in arrays.items():
        if t is not None and t.shape[0] != B:
            raise ValueError(f"{call}: {name} has {t.shape[0]} rows for {B} streams")


def _ptr(t):
    # ctypes turns None into NULL and an int into the pointer (argtypes c_void_p)
    return None if t is None else t.data_ptr()


def _stream():
    """The raw HIP stream of torch's current stream on the current device.
    torch's own accessor of the raw handle costs ~0.1 us against ~3 us for
    building a Stream object, which matters at small batch where a step is
    bounded by host time; the public API is the fallback."""
    torch = _torch()
    try:
        return torch._C._cuda_getCurrentRawStream(torch._C._cuda_getDevice())
    except AttributeError:
        return torch.cuda.current_stream().cuda_stream


class Workspace:
    """Device scratch for decode_attention's per-split partial results,
    cached per device and grown on demand.  Calls that share it must be
    ordered on one stream (torch's current stream is used for every call)."""

    _cache = {}

    @classmethod
    def get(cls, nbytes: int, device):
        torch = _torch()
        key = torch.device(device).index or 0
        buf = cls._cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device=device)
            cls._cache[key] = buf
        off = (-buf.data_ptr()) % 256
        return buf[off:]


def kv_cache_append(k_new, v_new, k_cache, v_cache, block_table, len_before, block_size=16):
    """k_new, v_new [B,T,H_kv,D]; k_cache [nb,H_kv,bs,D]; v_cache [nb,H_kv,D,bs];
    block_table [B,max_blocks] int32; len_before [B] int32.  In place."""
    torch = _torch()
    lib = load()
    _cuda("k_new", k_new, ndim=4)
    _cuda("v_new", v_new, k_new.dtype, 4)
    _cuda("k_cache", k_cache, k_new.dtype, 4)
    _cuda("v_cache", v_cache, k_new.dtype, 4)
    _cuda("block_table", block_table, torch.int32, 2)
    _cuda("len_before", len_before, torch.int32, 1)
    B, T, H, D = k_new.shape
    nb = k_cache.shape[0]
    if tuple(v_new.shape) != (B, T, H, D) or tuple(k_cache.shape) != (nb, H, block_size, D) \
            or tuple(v_cache.shape) != (nb, H, D, block_size):
        raise ValueError("kv_cache_append: shape mismatch")
    if block_table.shape[0] != B or len_before.shape[0] != B:
        raise ValueError("kv_cache_append: batch mismatch")
    _check("clm_kv_cache_append", lib.clm_kv_cache_append(
        _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        block_table.shape[1], _ptr(len_before), B, T, H, D, block_size, nb, _dt(k_new), _stream()))


def rope_kv_cache_append(q, k_new, v_new, k_cache, v_cache, block_table, len_before, positions,
                         rope_base, block_size=16):
    """kv_cache_append with rotary embedding at logical positions [B,T] int32
    applied to the new keys (as written) and to q [B,T,H_q,D] (in place)."""
    torch = _torch()
    lib = load()
    _cuda("q", q, ndim=4)
    _cuda("k_new", k_new, q.dtype, 4)
    _cuda("v_new", v_new, q.dtype, 4)
    _cuda("k_cache", k_cache, q.dtype, 4)
    _cuda("v_cache", v_cache, q.dtype, 4)
    _cuda("block_table", block_table, torch.int32, 2)
    _cuda("len_before", len_before, torch.int32, 1)
    _cuda("positions", positions, torch.int32, 2)
    B, T, H, D = k_new.shape
    H_q = q.shape[2]
    nb = k_cache.shape[0]
    if tuple(q.shape) != (B, T, H_q, D) or tuple(v_new.shape) != (B, T, H, D) \
            or tuple(k_cache.shape) != (nb, H, block_size, D) or tuple(v_cache.shape) != (nb, H, D, block_size) \
            or tuple(positions.shape) != (B, T):
        raise ValueError("rope_kv_cache_append: shape mismatch")
    if block_table.shape[0] != B or len_before.shape[0] != B:
        raise ValueError("rope_kv_cache_append: batch mismatch")
    _check("clm_rope_kv_cache_append", lib.clm_rope_kv_cache_append(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        block_table.shape[1], _ptr(len_before), _ptr(positions), C.c_float(rope_base), B, T, H_q, H, D,
        block_size, nb, _dt(k_new), _stream()))


def kv_cache_append_fp8(k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, len_before,
                        block_size=16):
    """E4M3 cache append: k_new, v_new [B,T,H_kv,D] bf16; k_cache
    [nb,H_kv,D/8,bs,8] and v_cache [nb,H_kv,D,bs] uint8; k_scale, v_scale
    [nb,H_kv,bs] float32.  In place."""
    torch = _torch()
    lib = load()
    _cuda("k_new", k_new, torch.bfloat16, 4)
    _cuda("v_new", v_new, torch.bfloat16, 4)
    _cuda("k_cache", k_cache, torch.uint8, 5)
    _cuda("v_cache", v_cache, torch.uint8, 4)
    _cuda("k_scale", k_scale, torch.float32, 3)
    _cuda("v_scale", v_scale, torch.float32, 3)
    _cuda("block_table", block_table, torch.int32, 2)
    _cuda("len_before", len_before, torch.int32, 1)
    B, T, H, D = k_new.shape
    nb = k_cache.shape[0]
    if tuple(v_new.shape) != (B, T, H, D) or tuple(k_cache.shape) != (nb, H, D // 8, block_size, 8) \
            or tuple(v_cache.shape) != (nb, H, D, block_size) or tuple(k_scale.shape) != (nb, H, block_size) \
            or tuple(v_scale.shape) != (nb, H, block_size):
        raise ValueError("kv_cache_append_fp8: shape mismatch")
    _rows("kv_cache_append_fp8", B, block_table=block_table, len_before=len_before)
    _check("clm_kv_cache_append_fp8", lib.clm_kv_cache_append_fp8(
        _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        block_table.shape[1], _ptr(len_before), B, T, H, D, block_size, nb, _stream()))


def rope_kv_cache_append_fp8(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, len_before,
                             positions, rope_base, block_size=16):
    """kv_cache_append_fp8 with the rotary embedding of rope_kv_cache_append:
    keys rotated (fp32) then quantized, q [B,T,H_q,D] bf16 rotated in place,
    values quantized unrotated.  positions [B,T] int32."""
    torch = _torch()
    lib = load()
    _cuda("q", q, torch.bfloat16, 4)
    _cuda("k_new", k_new, torch.bfloat16, 4)
    _cuda("v_new", v_new, torch.bfloat16, 4)
    _cuda("k_cache", k_cache, torch.uint8, 5)
    _cuda("v_cache", v_cache, torch.uint8, 4)
    _cuda("k_scale", k_scale, torch.float32, 3)
    _cuda("v_scale", v_scale, torch.float32, 3)
    _cuda("block_table", block_table, torch.int32, 2)
    _cuda("len_before", len_before, torch.int32, 1)
    _cuda("positions", positions, torch.int32, 2)
    B, T, H, D = k_new.shape
    H_q = q.shape[2]
    nb = k_cache.shape[0]
    if tuple(q.shape) != (B, T, H_q, D) or tuple(v_new.shape) != (B, T, H, D) \
            or tuple(k_cache.shape) != (nb, H, D // 8, block_size, 8) or tuple(v_cache.shape) != (nb, H, D, block_size) \
            or tuple(k_scale.shape) != (nb, H, block_size) or tuple(v_scale.shape) != (nb, H, block_size) \
            or tuple(positions.shape) != (B, T):
        raise ValueError("rope_kv_cache_append_fp8: shape mismatch")
    _rows("rope_kv_cache_append_fp8", B, block_table=block_table, len_before=len_before)
    _check("clm_rope_kv_cache_append_fp8", lib.clm_rope_kv_cache_append_fp8(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_table), block_table.shape[1], _ptr(len_before), _ptr(positions), C.c_float(rope_base), B, T,
        H_q, H, D, block_size, nb, _stream()))


@functools.lru_cache(maxsize=256)
def decode_attention_workspace_size(B, Kq, H_q, H_kv, D, max_kv_len) -> int:
    return int(load().clm_decode_attention_workspace_size(B, Kq, H_q, H_kv, D, max_kv_len))


def decode_attention(q, k_cache, v_cache, block_table, kv_len, max_kv_len, scale=None,
                     out=None, workspace=None, block_size=16):
    """q [B,Kq,H_q,D]; cache as for kv_cache_append; kv_len [B] int32 (keys
    seen by the last query, after this step's append).  Returns o [B,Kq,H_q,D]."""
    torch = _torch()
    lib = load()
    _cuda("q", q, ndim=4)
    _cuda("k_cache", k_cache, q.dtype, 4)
    _cuda("v_cache", v_cache, q.dtype, 4)
    _cuda("block_table", block_table, torch.int32, 2)
    _cuda("kv_len", kv_len, torch.int32, 1)
    B, Kq, H_q, D = q.shape
    nb, H_kv = k_cache.shape[0], k_cache.shape[1]
    if tuple(k_cache.shape) != (nb, H_kv, block_size, D) or tuple(v_cache.shape) != (nb, H_kv, D, block_size):
        raise ValueError("decode_attention: cache shape mismatch")
    _rows("decode_attention", B, block_table=block_table, kv_len=kv_len)
    if out is None:
        out = torch.empty_like(q)
    else:
        _out("out", out, q.shape, q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = decode_attention_workspace_size(B, Kq, H_q, H_kv, D, max_kv_len)
    if need == 0:
        raise ClmError("clm_decode_attention_workspace_size", -1)
    if workspace is None:
        workspace = Workspace.get(need, q.device)
    _check("clm_decode_attention", lib.clm_decode_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1], _ptr(kv_len),
        int(max_kv_len), _ptr(out), B, Kq, H_q, H_kv, D, block_size, nb, C.c_float(scale), _dt(q),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return out


def decode_attention_noalloc(q, k_cache, v_cache, block_table, kv_len, max_kv_len, scale=None, out=None,
                             block_size=16):
    """decode_attention without a workspace: the library's static 32 MiB
    per-GPU scratch holds the split partials, so the call allocates no device
    memory (``out`` must then be given by the caller).  Calls that overlap on
    one GPU race on that scratch."""
    torch = _torch()
    lib = load()
    _cuda("q", q, ndim=4)
    _cuda("k_cache", k_cache, q.dtype, 4)
    _cuda("v_cache", v_cache, q.dtype, 4)
    _cuda("block_table", block_table, torch.int32, 2)
    _cuda("kv_len", kv_len, torch.int32, 1)
    B, Kq, H_q, D = q.shape
    nb, H_kv = k_cache.shape[0], k_cache.shape[1]
    if tuple(k_cache.shape) != (nb, H_kv, block_size, D) or tuple(v_cache.shape) != (nb, H_kv, D, block_size):
        raise ValueError("decode_attention_noalloc: cache shape mismatch")
    _rows("decode_attention_noalloc", B, block_table=block_table, kv_len=kv_len)
    if out is None:
        raise ValueError("decode_attention_noalloc: the caller provides `out` (nothing is allocated here)")
    _out("out", out, q.shape, q.dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check("clm_decode_attention_noalloc", lib.clm_decode_attention_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), block_table.shape[1], _ptr(kv_len),
        int(max_kv_len), _ptr(out), B, Kq, H_q, H_kv, D, block_size, nb, C.c_float(scale), _dt(q), _stream()))
    return out


def decode_attention_fp8(q, k_cache, v_cache, k_scale, v_scale, block_table, kv_len, max_kv_len, scale=None,
                         out=None, workspace=None):
    """Attention over the E4M3 cache: q [B,Kq,H_q,D] bf16; caches uint8 and
    scales float32 as kv_cache_append_fp8.  Returns o [B,Kq,H_q,D] bf16."""
    torch = _torch()
    lib = load()
    _cuda("q", q, torch.bfloat16, 4)
    _cuda("k_cache", k_cache, torch.uint8, 5)
    _cuda("v_cache", v_cache, torch.uint8, 4)
    _cuda("k_scale", k_scale, torch.float32, 3)
    _cuda("v_scale", v_scale, torch.float32, 3)
    _cuda("block_table", block_table, torch.int32, 2)
    _cuda("kv_len", kv_len, torch.int32, 1)
    B, Kq, H_q, D = q.shape
    nb, H_kv, _, bs, _ = k_cache.shape
    if tuple(k_cache.shape) != (nb, H_kv, D // 8, bs, 8) or tuple(v_cache.shape) != (nb, H_kv, D, bs) \
            or tuple(k_scale.shape) != (nb, H_kv, bs) or tuple(v_scale.shape) != (nb, H_kv, bs):
        raise ValueError("decode_attention_fp8: shape mismatch")
    _rows("decode_attention_fp8", B, block_table=block_table, kv_len=kv_len)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _out("out", out, q.shape, torch.bfloat16)
    need = decode_attention_workspace_size(B, Kq, H_q, H_kv, D, max_kv_len)
    if need == 0:
        raise ClmError("clm_decode_attention_workspace_size", -1)
    if workspace is None:
        workspace = Workspace.get(need, q.device)
    _check("clm_decode_attention_fp8", lib.clm_decode_attention_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        block_table.shape[1], _ptr(kv_len), int(max_kv_len), _ptr(out), B, Kq, H_q, H_kv, D, bs, nb,
        C.c_float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
    return out


@functools.lru_cache(maxsize=256)
def codebook_head_workspace_size(M, d, V, G, bf16=True) -> int:
    return int(load().clm_codebook_head_workspace_size(M, d, V, G, CLM_BF16 if bf16 else CLM_F32))


@functools.lru_cache(maxsize=256)
def codebook_head_mlp_workspace_size(M, d, F, V, G) -> int:
    return int(load().clm_codebook_head_mlp_workspace_size(M, d, F, V, G))


def _head_workspace(need, workspace, device):
    """The caller's workspace (checked by the library), or a cached one when
    the plan needs scratch and none was given, or none."""
    if workspace is not None:
        _cuda("workspace", workspace, _torch().uint8, 1)
        return workspace
    if need == 0:
        return None
    return Workspace.get(need, device)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def codebook_head(h, W, head_id=None, out=None, workspace=None):
    """h [M,d]; W a [G,V,d] tensor or a list of G [V,d] tensors; head_id [M]
    int32 (required when G > 1).  Returns logits [M,V] float32."""
    torch = _torch()
    lib = load()
    _cuda("h", h, ndim=2)
    Ws = [W[g] for g in range(W.shape[0])] if isinstance(W, torch.Tensor) and W.dim() == 3 else list(W)
    for i, w in enumerate(Ws):
        _cuda(f"W[{i}]", w, h.dtype, 2)
    G = len(Ws)
    V, d = Ws[0].shape
    M = h.shape[0]
    if h.shape[1] != d or any(tuple(w.shape) != (V, d) for w in Ws):
        raise ValueError("codebook_head: shape mismatch")
    if head_id is not None:
        _cuda("head_id", head_id, torch.int32, 1)
        _rows("codebook_head", M, head_id=head_id)
    if out is None:
        out = torch.empty((M, V), dtype=torch.float32, device=h.device)
    else:
        _out("out", out, (M, V), torch.float32)
    arr = (C.c_void_p * G)(*[w.data_ptr() for w in Ws])
    ws = _head_workspace(codebook_head_workspace_size(M, d, V, G, h.dtype == torch.bfloat16), workspace,
                         h.device)
    _check("clm_codebook_head", lib.clm_codebook_head(
        _ptr(h), arr, G, _ptr(head_id), _ptr(out), M, d, V, _dt(h), _ptr(ws), _nbytes(ws), _stream()))
    return out


def codebook_head_mlp(h, W1, W2, head_id=None, act=None, out=None, workspace=None):
    """Two-layer head: h [M,d] bf16; W1 a [G,F,d] tensor or list of G [F,d];
    W2 a [G,V,F] tensor or list of G [V,F]; head_id [M] int32 (required when
    G > 1); act [M,F] bf16 scratch for the widened activation (allocated when
    None).  Returns (logits [M,V] float32, act)."""
    torch = _torch()
    lib = load()
    _cuda("h", h, torch.bfloat16, 2)

    def as_list(W):
        return [W[g] for g in range(W.shape[0])] if isinstance(W, torch.Tensor) and W.dim() == 3 else list(W)
    W1s, W2s = as_list(W1), as_list(W2)
    if len(W1s) != len(W2s):
        raise ValueError("codebook_head_mlp: W1 and W2 need one matrix per stage each")
    for i, (a, b) in enumerate(zip(W1s, W2s)):
        _cuda(f"W1[{i}]", a, torch.bfloat16, 2)
        _cuda(f"W2[{i}]", b, torch.bfloat16, 2)
    G = len(W1s)
    F, d = W1s[0].shape
    V = W2s[0].shape[0]
    M = h.shape[0]
    if h.shape[1] != d or any(tuple(w.shape) != (F, d) for w in W1s) or any(tuple(w.shape) != (V, F) for w in W2s):
        raise ValueError("codebook_head_mlp: shape mismatch")
    if head_id is not None:
        _cuda("head_id", head_id, torch.int32, 1)
        _rows("codebook_head_mlp", M, head_id=head_id)
    if act is None:
        act = torch.empty((M, F), dtype=torch.bfloat16, device=h.device)
    else:
        _out("act", act, (M, F), torch.bfloat16)
    if out is None:
        out = torch.empty((M, V), dtype=torch.float32, device=h.device)
    else:
        _out("out", out, (M, V), torch.float32)
    a1 = (C.c_void_p * G)(*[w.data_ptr() for w in W1s])
    a2 = (C.c_void_p * G)(*[w.data_ptr() for w in W2s])
    ws = _head_workspace(codebook_head_mlp_workspace_size(M, d, F, V, G), workspace, h.device)
    _check("clm_codebook_head_mlp", lib.clm_codebook_head_mlp(
        _ptr(h), a1, a2, G, _ptr(head_id), _ptr(act), _ptr(out), M, d, F, V, _dt(h), _ptr(ws), _nbytes(ws),
        _stream()))
    return out, act


def sample_or_argmax(logits, temperature=None, uniforms=None, vocab_valid=None, out=None):
    """logits [M,V] float32 (rows may be padded: ld = stride); temperature,
    uniforms [M] float32; vocab_valid [M] int32.  Returns tokens [M] int32."""
    torch = _torch()
    lib = load()
    if logits.dim() != 2 or logits.dtype != torch.float32 or not logits.is_cuda or logits.stride(1) != 1:
        raise ValueError("logits must be a 2-D float32 GPU tensor with unit column stride")
    M, V = logits.shape
    for name, t, dt in (("temperature", temperature, torch.float32), ("uniforms", uniforms, torch.float32),
                        ("vocab_valid", vocab_valid, torch.int32)):
        if t is not None:
            _cuda(name, t, dt, 1)
            if t.shape[0] != M:
                raise ValueError(f"{name} must have {M} entries (one per row), got {t.shape[0]}")
    if out is None:
        out = torch.empty(M, dtype=torch.int32, device=logits.device)
    else:
        _out("out", out, (M,), torch.int32)
    _check("clm_sample_or_argmax", lib.clm_sample_or_argmax(
        _ptr(logits), M, V, logits.stride(0), _ptr(temperature), _ptr(uniforms), _ptr(vocab_valid),
        _ptr(out), _stream()))
    return out


def spec_verify(target_logits, draft_probs, draft_tokens, u_accept, u_resample, temperature,
                out_tokens=None, num_emitted=None):
    """target_logits, draft_probs [B,K,V] float32; draft_tokens [B,K] int32;
    u_accept [B,K], u_resample [B] float32.  Returns (out_tokens [B,K] int32
    padded with -1, num_emitted [B] int32)."""
    torch = _torch()
    lib = load()
    _cuda("target_logits", target_logits, torch.float32, 3)
    _cuda("draft_probs", draft_probs, torch.float32, 3)
    _cuda("draft_tokens", draft_tokens, torch.int32, 2)
    _cuda("u_accept", u_accept, torch.float32, 2)
    _cuda("u_resample", u_resample, torch.float32, 1)
    B, K, V = target_logits.shape
    if tuple(draft_probs.shape) != (B, K, V) or tuple(draft_tokens.shape) != (B, K) \
            or tuple(u_accept.shape) != (B, K) or tuple(u_resample.shape) != (B,):
        raise ValueError("spec_verify: shape mismatch")
    if out_tokens is None:
        out_tokens = torch.empty((B, K), dtype=torch.int32, device=target_logits.device)
    else:
        _out("out_tokens", out_tokens, (B, K), torch.int32)
    if num_emitted is None:
        num_emitted = torch.empty(B, dtype=torch.int32, device=target_logits.device)
    else:
        _out("num_emitted", num_emitted, (B,), torch.int32)
    _check("clm_spec_verify", lib.clm_spec_verify(
        _ptr(target_logits), _ptr(draft_probs), _ptr(draft_tokens), _ptr(u_accept), _ptr(u_resample),
        C.c_float(temperature), B, K, V, _ptr(out_tokens), _ptr(num_emitted), _stream()))
    return out_tokens, num_emitted


def spec_verify_bonus(target_logits, draft_probs, draft_tokens, u_accept, u_resample, temperature,
                      out_tokens=None, num_emitted=None):
    """target_logits [B,K+1,V], draft_probs [B,K,V] float32; draft_tokens
    [B,K] int32; u_accept [B,K], u_resample [B] float32.  Returns (out_tokens
    [B,K+1] int32 padded with -1, num_emitted [B] int32 in [1, K+1])."""
    torch = _torch()
    lib = load()
    _cuda("target_logits", target_logits, torch.float32, 3)
    _cuda("draft_probs", draft_probs, torch.float32, 3)
    _cuda("draft_tokens", draft_tokens, torch.int32, 2)
    _cuda("u_accept", u_accept, torch.float32, 2)
    _cuda("u_resample", u_resample, torch.float32, 1)
    B, K, V = draft_probs.shape
    if tuple(target_logits.shape) != (B, K + 1, V) or tuple(draft_tokens.shape) != (B, K) \
            or tuple(u_accept.shape) != (B, K) or tuple(u_resample.shape) != (B,):
        raise ValueError("spec_verify_bonus: shape mismatch")
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=target_logits.device)
    else:
        _out("out_tokens", out_tokens, (B, K + 1), torch.int32)
    if num_emitted is None:
        num_emitted = torch.empty(B, dtype=torch.int32, device=target_logits.device)
    else:
        _out("num_emitted", num_emitted, (B,), torch.int32)
    _check("clm_spec_verify_bonus", lib.clm_spec_verify_bonus(
        _ptr(target_logits), _ptr(draft_probs), _ptr(draft_tokens), _ptr(u_accept), _ptr(u_resample),
        C.c_float(temperature), B, K, V, _ptr(out_tokens), _ptr(num_emitted), _stream()))
    return out_tokens, num_emitted


def advance_lengths(len_before, kv_len, T_new, positions=None, num_emitted=None):
    """Device-side advance of every stream by num_emitted[b] (or T_new):
    len_before, kv_len [B] int32 and positions [B,T_new] int32, in place."""
    torch = _torch()
    lib = load()
    _cuda("len_before", len_before, torch.int32, 1)
    B = len_before.shape[0]
    _out("kv_len", kv_len, (B,), torch.int32)
    if positions is not None:
        _out("positions", positions, (B, T_new), torch.int32)
    if num_emitted is not None:
        _out("num_emitted", num_emitted, (B,), torch.int32)
    _check("clm_advance_lengths", lib.clm_advance_lengths(
        _ptr(len_before), _ptr(kv_len), _ptr(positions), _ptr(num_emitted), B, T_new, _stream()))


def pick_bucket(bucket_sizes, B) -> int:
    """Index of the smallest captured batch size >= B (clm_pick_bucket), or -1."""
    arr = (C.c_int32 * len(bucket_sizes))(*bucket_sizes)
    return int(load().clm_pick_bucket(C.cast(arr, C.c_void_p), len(bucket_sizes), int(B)))


class DecodeLoop:
    """n_steps decode steps captured as one HIP graph (clm_decode_loop_*).

    Per-step arrays carry a leading n_steps axis: k_new, v_new [n, B, Kq,
    H_kv, D]; q, o [n, B, Kq, H_q, D]; logits [n, B*Kq, V]; tokens,
    temperature, uniforms [n, B*Kq]; draft_probs [n, B, Kq, V]; draft_tokens,
    u_accept, out_tokens [n, B, Kq]; u_resample, num_emitted [n, B].  The
    cache, block table, lengths (and positions) are as for the single
    calls; the lengths and positions advance on the device after each step.
    With k_scale / v_scale the cache is FP8 (E4M3) as for
    kv_cache_append_fp8 (uint8 k_cache [nb, H_kv, D/8, bs, 8], v_cache [nb,
    H_kv, D, bs], float32 scales [nb, H_kv, bs]); q, k_new and v_new are then
    bf16 and an attention workspace is required (with positions, the steps
    append by rope_kv_cache_append_fp8).
    With W2 the head has two layers (codebook_head_mlp): W holds the first
    layer [G, F, H_q*D] and W2 the second [G, V, F], bf16; act [B*Kq, F] bf16
    is the activation scratch (allocated when None).
    mode: "greedy", "sample", "spec" or "spec_bonus" (verification with a
    bonus token: the Kq queries score the last kept token and Kq - 1 drafts,
    so draft_probs is [n, B, Kq-1, V], draft_tokens and u_accept [n, B,
    Kq-1], out_tokens [n, B, Kq]).  Every tensor must stay alive while
    the loop exists (this object keeps references); launch() enqueues all
    n_steps steps on torch's current stream."""

    _MODES = {"greedy": 0, "sample": 1, "spec": 2, "spec_bonus": 3}

    def __init__(self, *, k_cache, v_cache, block_table, len_before, kv_len, max_kv_len, k_new, v_new, q, W, o,
                 logits, head_id=None, positions=None, rope_base=1.0e6, mode="greedy", tokens=None,
                 temperature=None, uniforms=None, spec_temperature=0.0, draft_probs=None, draft_tokens=None,
                 u_accept=None, u_resample=None, out_tokens=None, num_emitted=None, attn_workspace=None,
                 block_size=16, k_scale=None, v_scale=None, W2=None, act=None):
        torch = _torch()
        self._lib = load()
        self._h = None
        n, B, Kq, H_q, D = q.shape
        dt = q.dtype
        for name, t in (("k_new", k_new), ("v_new", v_new)):
            _cuda(name, t, dt, 5)
        H_kv = k_new.shape[3]
        if tuple(k_new.shape) != (n, B, Kq, H_kv, D) or tuple(v_new.shape) != (n, B, Kq, H_kv, D):
            raise ValueError("DecodeLoop: k_new/v_new shape")
        _cuda("q", q, dt, 5)
        _out("o", o, q.shape, dt)
        nb = k_cache.shape[0]
        if (k_scale is None) != (v_scale is None):
            raise ValueError("DecodeLoop: k_scale and v_scale go together")
        if k_scale is not None:
            if dt != torch.bfloat16 or D % 8:
                raise ValueError("DecodeLoop: an FP8 cache takes bf16 queries and rows, D a multiple of 8")
            _out("k_cache", k_cache, (nb, H_kv, D // 8, block_size, 8), torch.uint8)
            _out("v_cache", v_cache, (nb, H_kv, D, block_size), torch.uint8)
            _out("k_scale", k_scale, (nb, H_kv, block_size), torch.float32)
            _out("v_scale", v_scale, (nb, H_kv, block_size), torch.float32)
        else:
            _out("k_cache", k_cache, (nb, H_kv, block_size, D), dt)
            _out("v_cache", v_cache, (nb, H_kv, D, block_size), dt)
        _cuda("block_table", block_table, torch.int32, 2)
        if block_table.shape[0] != B:
            raise ValueError("DecodeLoop: block_table rows")
        _out("len_before", len_before, (B,), torch.int32)
        _out("kv_len", kv_len, (B,), torch.int32)
        if positions is not None:
            _out("positions", positions, (B, Kq), torch.int32)
        Ws = [W[g] for g in range(W.shape[0])] if isinstance(W, torch.Tensor) and W.dim() == 3 else list(W)
        G = len(Ws)
        M = B * Kq
        W2s, F = None, 0
        if W2 is not None:
            if dt != torch.bfloat16:
                raise ValueError("DecodeLoop: the two-layer head takes bf16")
            W2s = [W2[g] for g in range(W2.shape[0])] if isinstance(W2, torch.Tensor) and W2.dim() == 3 \
                else list(W2)
            if len(W2s) != G:
                raise ValueError("DecodeLoop: W and W2 need one matrix per stage each")
            F, V = Ws[0].shape[0], W2s[0].shape[0]
            for i, (a, b2) in enumerate(zip(Ws, W2s)):
                _out(f"W[{i}]", a, (F, H_q * D), dt)
                _out(f"W2[{i}]", b2, (V, F), dt)
            if act is None:
                act = torch.empty((M, F), dtype=torch.bfloat16, device=q.device)
            _out("act", act, (M, F), torch.bfloat16)
        else:
            V = Ws[0].shape[0]
            for i, w in enumerate(Ws):
                _out(f"W[{i}]", w, (V, H_q * D), dt)
        _out("logits", logits, (n, M, V), torch.float32)
        if head_id is not None:
            _out("head_id", head_id, (M,), torch.int32)
        if mode not in self._MODES:
            raise ValueError(f"DecodeLoop: mode {mode!r}")
        if mode in ("greedy", "sample"):
            _out("tokens", tokens, (n, M), torch.int32)
        if mode == "sample":
            _out("temperature", temperature, (n, M), torch.float32)
            _out("uniforms", uniforms, (n, M), torch.float32)
        if mode in ("spec", "spec_bonus"):
            Kd = Kq - 1 if mode == "spec_bonus" else Kq
            if Kd < 1:
                raise ValueError("DecodeLoop: spec_bonus needs Kq >= 2 (the last kept token and a draft)")
            _out("draft_probs", draft_probs, (n, B, Kd, V), torch.float32)
            _out("draft_tokens", draft_tokens, (n, B, Kd), torch.int32)
            _out("u_accept", u_accept, (n, B, Kd), torch.float32)
            _out("u_resample", u_resample, (n, B), torch.float32)
            _out("out_tokens", out_tokens, (n, B, Kq), torch.int32)
            _out("num_emitted", num_emitted, (n, B), torch.int32)
        if attn_workspace is not None:
            _cuda("attn_workspace", attn_workspace, torch.uint8, 1)
        self._warr = (C.c_void_p * G)(*[w.data_ptr() for w in Ws])
        self._w2arr = None if W2s is None else (C.c_void_p * G)(*[w.data_ptr() for w in W2s])
        self._keep = [k_cache, v_cache, block_table, len_before, kv_len, positions, k_new, v_new, q, Ws, head_id,
                      o, logits, tokens, temperature, uniforms, draft_probs, draft_tokens, u_accept, u_resample,
                      out_tokens, num_emitted, attn_workspace, k_scale, v_scale, W2s, act]
        p = lambda t: 0 if t is None else t.data_ptr()
        d = _lib.DecodeStepDesc(
            B=B, Kq=Kq, H_q=H_q, H_kv=H_kv, D=D, block_size=block_size, num_blocks=nb,
            max_blocks=block_table.shape[1], max_kv_len=int(max_kv_len), G=G, V=V, dt=_dt(q),
            k_cache=p(k_cache), v_cache=p(v_cache), block_table=p(block_table), len_before=p(len_before),
            kv_len=p(kv_len), positions=p(positions), rope_base=float(rope_base), k_new=p(k_new), v_new=p(v_new),
            q=p(q), W=C.cast(self._warr, C.c_void_p).value, head_id=p(head_id), o=p(o), logits=p(logits),
            attn_workspace=p(attn_workspace), attn_workspace_bytes=_nbytes(attn_workspace),
            mode=self._MODES[mode], temperature=p(temperature), uniforms=p(uniforms), tokens=p(tokens),
            spec_temperature=float(spec_temperature), draft_probs=p(draft_probs), draft_tokens=p(draft_tokens),
            u_accept=p(u_accept), u_resample=p(u_resample), out_tokens=p(out_tokens), num_emitted=p(num_emitted),
            k_scale=p(k_scale), v_scale=p(v_scale),
            W2=None if W2s is None else C.cast(self._w2arr, C.c_void_p).value, F=F, act=p(act))
        h = C.c_void_p()
        _check("clm_decode_loop_create", self._lib.clm_decode_loop_create(C.byref(d), n, C.byref(h)))
        self._h = h
        self.n_steps = n

    def launch(self):
        if self._h is None:
            raise RuntimeError("DecodeLoop: closed")
        _check("clm_decode_loop_launch", self._lib.clm_decode_loop_launch(self._h, _stream()))

    def close(self):
        if self._h is not None:
            _check("clm_decode_loop_destroy", self._lib.clm_decode_loop_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
