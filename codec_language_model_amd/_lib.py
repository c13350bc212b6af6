"""ctypes declarations for libclm.so (include/clm.h).  Marshalling only."""

from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libclm.so")

CLM_F32 = 0
CLM_BF16 = 1

STATUS = {
    0: "CLM_OK",
    -1: "CLM_ERR_INVALID_ARG",
    -2: "CLM_ERR_UNSUPPORTED",
    -3: "CLM_ERR_CAPACITY",
    -4: "CLM_ERR_WORKSPACE",
    -5: "CLM_ERR_HIP",
    -6: "CLM_ERR_DEVICE_DATA",
}

_vp = C.c_void_p
_i = C.c_int
_f = C.c_float
_sz = C.c_size_t

# name -> (restype, argtypes); order and types follow include/clm.h
SIGNATURES = {
    "clm_status_string": (C.c_char_p, [_i]),
    "clm_version": (_i, []),
    "clm_set_checked": (_i, [_i]),
    "clm_kv_cache_append": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "clm_rope_kv_cache_append": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _f, _i, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "clm_decode_attention_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i]),
    "clm_decode_attention": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i,
                                  _f, _i, _vp, _sz, _vp]),
    "clm_decode_attention_noalloc": (_i, [_vp, _vp, _vp, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i,
                                          _f, _i, _vp]),
    "clm_kv_cache_append_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "clm_rope_kv_cache_append_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _f, _i, _i, _i, _i,
                                          _i, _i, _i, _vp]),
    "clm_decode_attention_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i,
                                      _f, _vp, _sz, _vp]),
    "clm_codebook_head_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "clm_codebook_head": (_i, [_vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "clm_codebook_head_mlp_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "clm_codebook_head_mlp": (_i, [_vp, _vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _sz, _vp]),
    "clm_sample_or_argmax": (_i, [_vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "clm_spec_verify": (_i, [_vp, _vp, _vp, _vp, _vp, _f, _i, _i, _i, _vp, _vp, _vp]),
    "clm_spec_verify_bonus": (_i, [_vp, _vp, _vp, _vp, _vp, _f, _i, _i, _i, _vp, _vp, _vp]),
}



class DecodeStepDesc(C.Structure):
    """clm_decode_step_desc (include/clm.h), field for field."""
    _fields_ = [
        ("B", _i), ("Kq", _i), ("H_q", _i), ("H_kv", _i), ("D", _i),
        ("block_size", _i), ("num_blocks", _i), ("max_blocks", _i), ("max_kv_len", _i),
        ("G", _i), ("V", _i), ("dt", _i),
        ("k_cache", _vp), ("v_cache", _vp), ("block_table", _vp), ("len_before", _vp), ("kv_len", _vp),
        ("positions", _vp), ("rope_base", _f),
        ("k_new", _vp), ("v_new", _vp), ("q", _vp), ("W", _vp), ("head_id", _vp),
        ("o", _vp), ("logits", _vp), ("attn_workspace", _vp), ("attn_workspace_bytes", _sz),
        ("mode", _i), ("temperature", _vp), ("uniforms", _vp), ("tokens", _vp),
        ("spec_temperature", _f), ("draft_probs", _vp), ("draft_tokens", _vp), ("u_accept", _vp),
        ("u_resample", _vp), ("out_tokens", _vp), ("num_emitted", _vp),
        ("k_scale", _vp), ("v_scale", _vp), ("W2", _vp), ("F", _i), ("act", _vp),
    ]


SIGNATURES.update({
    "clm_advance_lengths": (_i, [_vp, _vp, _vp, _vp, _i, _i, _vp]),
    "clm_decode_loop_create": (_i, [C.POINTER(DecodeStepDesc), _i, C.POINTER(_vp)]),
    "clm_decode_loop_launch": (_i, [_vp, _vp]),
    "clm_decode_loop_destroy": (_i, [_vp]),
    "clm_pick_bucket": (_i, [_vp, _i, _i]),
})

_lib = None


def load(path: str = None) -> C.CDLL:
    """Load libclm.so (once): ``path``, else $CLM_LIBRARY, else the in-tree
    build.  Raises if the library is missing: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("CLM_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m codec_language_model_amd.build` "
            "(or __graft_entry__.build()); there is no CPU fallback")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
