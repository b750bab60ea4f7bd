"""ctypes view of libgqa.so, the C ABI declared in include/gqa.h. No torch here.

The library is built in-tree by ``python attention_head_qk_amd/build.py``. Loading fails
loudly (ImportError) when it is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa.so")

GQA_OK, GQA_EINVAL, GQA_ENOTSUP, GQA_EWORKSPACE, GQA_EHIP = range(5)
GQA_F32, GQA_BF16 = 0, 1
GQA_OP_PREFILL, GQA_OP_DECODE, GQA_OP_QK_NORM_ROPE = 0, 1, 2
GQA_ROPE_BASE, GQA_ROPE_LINEAR, GQA_ROPE_YARN, GQA_ROPE_NTK = range(4)
GQA_DECODE_NOALLOC_MAX_BYTES = 64 * 1024 * 1024

# Every function include/gqa.h declares, with its ctypes signature.
_vp = ctypes.c_void_p
_i = ctypes.c_int


class GqaParams(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int),
        ("q_norm_w", _vp),
        ("k_norm_w", _vp),
        ("eps", ctypes.c_float),
        ("rope_theta", ctypes.c_double),
        ("scale", ctypes.c_float),
        ("cu_seqlens", _vp),
        ("k_out", _vp),
        ("k_new", _vp),
        ("v_new", _vp),
        ("positions", _vp),
        ("workspace", _vp),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", _vp),
        ("prof_start", _vp),
        ("prof_stop", _vp),
        ("window", ctypes.c_int),
        ("block_mask", _vp),
        ("block_mask_words", ctypes.c_int),
        ("rope_inv_freq", ctypes.POINTER(ctypes.c_double)),
    ]


SIGNATURES = {
    "gqa_params_init": (None, [ctypes.POINTER(GqaParams)]),
    "gqa_prefill": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, ctypes.POINTER(GqaParams)]),
    "gqa_prefill_cached": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                                ctypes.POINTER(GqaParams)]),
    "gqa_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, ctypes.POINTER(GqaParams)]),
    "gqa_decode_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, ctypes.POINTER(GqaParams)]),
    "gqa_decode_graph_create": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                     ctypes.POINTER(GqaParams), ctypes.POINTER(_vp)]),
    "gqa_decode_graph_create_steps": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                           ctypes.POINTER(GqaParams), ctypes.POINTER(_vp)]),
    "gqa_decode_graph_launch": (_i, [_vp, _vp]),
    "gqa_decode_graph_destroy": (_i, [_vp]),
    "gqa_qk_norm_rope": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, ctypes.POINTER(GqaParams)]),
    "gqa_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i, _i, _i, _i]),
    "gqa_decode_split_keys": (_i, [_i, _i, _i, _i]),
    "gqa_rope_freq_table": (_i, [_i, _i, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                 ctypes.c_double, ctypes.c_double, ctypes.POINTER(ctypes.c_double)]),
    "gqa_status_str": (ctypes.c_char_p, [_i]),
}


class GqaError(RuntimeError):
    def __init__(self, code: int, fn: str):
        self.code = code
        super().__init__(f"{fn} failed: {status_str(code)}")


_LIB = None


def load() -> ctypes.CDLL:
    """Load libgqa.so once; raise ImportError if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python attention_head_qk_amd/build.py` (needs hipcc)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _LIB = lib
    return lib


def status_str(code: int) -> str:
    return load().gqa_status_str(code).decode()


def check(code: int, fn: str) -> None:
    if code != GQA_OK:
        raise GqaError(code, fn)


def default_params() -> GqaParams:
    p = GqaParams()
    load().gqa_params_init(ctypes.byref(p))
    return p
