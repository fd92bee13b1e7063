"""ctypes loader for libgqa_decode.so: symbol signatures and status codes.

Marshalling only. A missing library raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

F32 = 0
BF16 = 1

OK = 0
ERR_ARG = -1
ERR_GROUPS = -2
ERR_UNSUPPORTED = -3
ERR_CAPACITY = -4
ERR_WORKSPACE = -5
ERR_HIP = -6

PATH_AUTO = 0
PATH_VECTOR = 1
PATH_MATRIX = 2
MERGE_INLINE = 0x10  # OR into path: split segments merged inside the decode launch
MERGE_KERNEL = 0x20  # OR into path: split segments merged by a second launch
MERGE_SPREAD = 0x80  # OR into path: split segments merged by their parts at the end of the launch (stream kernel)
PLAN_STREAM = 0x40   # reported by gqa_decode_plan: the matrix path's one-block streaming kernel

ERROR_NAMES = {
    ERR_ARG: "GQA_ERR_ARG", ERR_GROUPS: "GQA_ERR_GROUPS", ERR_UNSUPPORTED: "GQA_ERR_UNSUPPORTED",
    ERR_CAPACITY: "GQA_ERR_CAPACITY", ERR_WORKSPACE: "GQA_ERR_WORKSPACE", ERR_HIP: "GQA_ERR_HIP",
}

# Every function include/gqa_decode.h declares, with its ctypes signature.
_vp, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
_ip = ctypes.POINTER(ctypes.c_int)
SIGNATURES = {
    "gqa_kv_append": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "gqa_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "gqa_decode_attention": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _f32, _i32, _vp, _sz, _vp]),
    "gqa_decode_attention_ex": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _f32, _i32, _vp, _sz, _vp, _i32, _i32]),
    "gqa_decode_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                               _f32, _i32, _vp, _sz, _vp]),
    "gqa_decode_step_ex": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                  _f32, _i32, _vp, _sz, _vp, _i32, _i32]),
    "gqa_decode_plan": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _ip, _ip]),
    "gqa_packed_weight_bytes": (_sz, [_i32, _i32]),
    "gqa_pack_weight": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp]),
    "gqa_linear": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "gqa_decode_layer": (_i32, [_vp] * 13 + [_i32] * 8 + [_f32, _i32, _vp, _sz, _vp]),
    "gqa_fold_kv_heads": (_i32, [_vp, _vp, _vp] + [_i32] * 8 + [_vp]),
    "gqa_kv_append_paged": (_i32, [_vp] * 6 + [_i32] * 9 + [_vp]),
    "gqa_decode_attention_paged": (_i32, [_vp] * 6 + [_i32] * 9 + [_f32, _i32, _vp, _sz, _vp]),
    "gqa_decode_step_paged": (_i32, [_vp] * 8 + [_i32] * 9 + [_f32, _i32, _vp, _sz, _vp]),
    "gqa_decode_multi_workspace_size": (_sz, [_i32] * 7),
    "gqa_kv_append_multi": (_i32, [_vp] * 5 + [_i32] * 8 + [_vp]),
    "gqa_decode_attention_multi": (_i32, [_vp] * 5 + [_i32] * 8 + [_f32, _i32, _vp, _sz, _vp]),
    "gqa_decode_step_multi": (_i32, [_vp] * 7 + [_i32] * 8 + [_f32, _i32, _vp, _sz, _vp]),
    "gqa_kv_append_multi_paged": (_i32, [_vp] * 6 + [_i32] * 10 + [_vp]),
    "gqa_decode_attention_multi_paged": (_i32, [_vp] * 6 + [_i32] * 10 + [_f32, _i32, _vp, _sz, _vp]),
    "gqa_decode_step_multi_paged": (_i32, [_vp] * 8 + [_i32] * 10 + [_f32, _i32, _vp, _sz, _vp]),
    "gqa_decode_step_static": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                      _f32, _i32, _vp]),
    "gqa_read_bandwidth": (_i32, [_vp, _sz, _vp, _i32, _vp]),
    "gqa_last_error": (ctypes.c_char_p, []),
}

_lib = None


class GqaError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn} returned {ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


def load(path: str = LIB_PATH):
    """Load the library once and attach the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with gqa_kv_cache_decode_amd.build.build() "
            "(or __graft_entry__.build()); there is no CPU fallback")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(code: int, fn: str) -> None:
    if code != OK:
        raise GqaError(code, fn, load().gqa_last_error().decode())
