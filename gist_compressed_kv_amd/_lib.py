"""ctypes view of libgist_attn.so (the C ABI declared in include/gist_attn.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgist_attn.so")

GIST_OK = 0
GIST_ERR_INVALID_ARG = -1
GIST_ERR_UNSUPPORTED = -2
GIST_ERR_OUT_OF_RANGE = -3
GIST_ERR_HIP = -4

GIST_F32 = 0
GIST_BF16 = 1
GIST_FP8_E4M3 = 2

STATUS_NAMES = {
    GIST_OK: "GIST_OK",
    GIST_ERR_INVALID_ARG: "GIST_ERR_INVALID_ARG",
    GIST_ERR_UNSUPPORTED: "GIST_ERR_UNSUPPORTED",
    GIST_ERR_OUT_OF_RANGE: "GIST_ERR_OUT_OF_RANGE",
    GIST_ERR_HIP: "GIST_ERR_HIP",
}

# Every symbol include/gist_attn.h declares: name -> (restype, argtypes)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t
class GistGroup(ctypes.Structure):
    """struct gist_group of include/gist_attn.h."""
    _fields_ = [("layer", _i32), ("P", _i32), ("item_ids", _vp), ("q_ids", _vp), ("q", _vp),
                ("k_new", _vp), ("v_new", _vp), ("out", _vp)]


SIGNATURES = {
    "gist_pool_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32]),
    "gist_pool_create": (_i32, [ctypes.POINTER(_vp), _i32, _i64, _i32, _i32, _i32, _i32, _vp, _sz]),
    "gist_pool_destroy": (_i32, [_vp]),
    "gist_pool_write": (_i32, [_vp, _i32, _vp, _i64, _vp, _vp, _i32, _f32, _vp]),
    "gist_attn_forward": (_i32, [_vp, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _f32,
                                 _f32, _vp, _vp, _vp, _vp]),
    "gist_attn_forward_paged": (_i32, [_vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32, _i32, _i32,
                                       _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _f32, _f32,
                                       _vp, _vp]),
    "gist_attn_forward_paged_fp8": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32,
                                           _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32,
                                           _f32, _f32, _vp, _vp]),
    "gist_attn_forward_last": (_i32, [_vp, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _i32,
                                      _f32, _f32, _vp, _vp, _vp, _vp]),
    "gist_attn_forward_grouped": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _f32, _vp]),
    "gist_prefill_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "gist_prefill_attn": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _f32,
                                 _f32, _vp, _vp, _sz, _vp, _i32, _vp, _vp]),
    "paged_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "paged_decode_attn": (_i32, [_vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp,
                                 _i32, _i32, _i32, _i32, _f32, _f32, _vp, _vp, _sz, _vp]),
    "paged_decode_attn_fp8": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32, _vp,
                                     _vp, _vp, _vp, _i32, _i32, _i32, _f32, _f32, _vp, _vp, _sz,
                                     _vp]),
    "paged_decode_attn_noalloc": (_i32, [_vp, _vp, _i64, _i32, _vp, _i32, _vp, _i32, _vp, _vp, _vp,
                                         _vp, _i32, _i32, _i32, _i32, _f32, _f32, _vp, _vp]),
    "gist_last_error": (ctypes.c_char_p, []),
}

_lib = None


class GistError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {message}")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m gist_compressed_kv_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(status: int, where: str) -> None:
    if status != GIST_OK:
        raise GistError(status, where, lib().gist_last_error().decode())
