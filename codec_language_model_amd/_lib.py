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
