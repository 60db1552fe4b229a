"""ctypes declarations of the C ABI in ``include/yoco.h``.

Loading is lazy and loud: the first use raises ``RuntimeError`` when
``libyoco.so`` has not been built; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libyoco.so")

YOCO_DT_F32 = 0
YOCO_DT_BF16 = 1
YOCO_MAX_SEQ = 256
YOCO_DECODE_COUNTER_BYTES = YOCO_MAX_SEQ * 64 * 4
YOCO_DECODE_NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024

STATUS = {
    0: "YOCO_OK", 1: "YOCO_ERR_NULL_POINTER", 2: "YOCO_ERR_BAD_SHAPE", 3: "YOCO_ERR_BAD_DTYPE",
    4: "YOCO_ERR_OUT_OF_RANGE", 5: "YOCO_ERR_WORKSPACE", 6: "YOCO_ERR_HIP", 7: "YOCO_ERR_BAD_VALUE",
    8: "YOCO_ERR_ALIGNMENT",
}


class YocoError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class KVCacheStruct(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("len_host", ctypes.POINTER(ctypes.c_int64)),
        ("seq_capacity", ctypes.c_int64),
        ("n_seq", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("row_stride", ctypes.c_int64),
    ]


_lock = threading.Lock()
_lib = None


def _declare(lib):
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    cp = ctypes.POINTER(KVCacheStruct)
    st = ctypes.c_int
    lib.yoco_abi_version.restype = ctypes.c_int
    lib.yoco_abi_version.argtypes = []
    lib.yoco_last_error.restype = ctypes.c_char_p
    lib.yoco_last_error.argtypes = []
    lib.yoco_kv_cache_bytes.restype = st
    lib.yoco_kv_cache_bytes.argtypes = [i32, i64, i32, i32, i32, i64, ctypes.POINTER(sz)]
    lib.yoco_kv_cache_row_stride.restype = st
    lib.yoco_kv_cache_row_stride.argtypes = [i32, i32, i32, ctypes.POINTER(i64)]
    lib.yoco_kv_project.restype = st
    lib.yoco_kv_project.argtypes = [vp, i32, i64, i32, vp, f32, vp, vp, i32, cp, i32, i64, vp, sz, vp]
    lib.yoco_kv_append.restype = st
    lib.yoco_kv_append.argtypes = [vp, i32, i32, vp, f32, vp, vp, i32, cp, vp, sz, vp]
    lib.yoco_q_project.restype = st
    lib.yoco_q_project.argtypes = [vp, i32, i64, i32, vp, f32, vp, i32, i32, i32, vp, i32, vp, sz, vp]
    lib.yoco_project_workspace.restype = st
    lib.yoco_project_workspace.argtypes = [i64, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.yoco_fold_norm_gain.restype = st
    lib.yoco_fold_norm_gain.argtypes = [vp, i32, vp, i32, i32, vp, vp]
    lib.yoco_default_softmax_scale.restype = st
    lib.yoco_default_softmax_scale.argtypes = [i32, ctypes.POINTER(f32)]
    f64 = ctypes.c_double
    lib.yoco_kv_project_rope.restype = st
    lib.yoco_kv_project_rope.argtypes = [vp, i32, i64, i32, vp, f32, vp, vp, i32, cp, i32, i64, f64, vp, sz, vp]
    lib.yoco_kv_append_rope.restype = st
    lib.yoco_kv_append_rope.argtypes = [vp, i32, i32, vp, f32, vp, vp, i32, cp, f64, vp, sz, vp]
    lib.yoco_q_project_rope.restype = st
    lib.yoco_q_project_rope.argtypes = [vp, i32, i64, i32, vp, f32, vp, i32, i32, i32, vp, i32, vp, i64, f64, vp,
                                        sz, vp]
    lib.yoco_cross_attn_prefill.restype = st
    lib.yoco_cross_attn_prefill.argtypes = [vp, i32, i64, i64, i32, cp, i32, f32, vp, i32, vp, vp]
    lib.yoco_cross_attn_prefill_bwd_workspace.restype = st
    lib.yoco_cross_attn_prefill_bwd_workspace.argtypes = [i64, i32, ctypes.POINTER(sz)]
    lib.yoco_cross_attn_prefill_bwd.restype = st
    lib.yoco_cross_attn_prefill_bwd.argtypes = [vp, vp, i32, vp, vp, i64, i64, i32, cp, i32, f32, vp, vp, vp,
                                                vp, sz, vp]
    lib.yoco_project_bwd_workspace.restype = st
    lib.yoco_project_bwd_workspace.argtypes = [i64, i32, i32, i32, ctypes.POINTER(sz)]
    lib.yoco_kv_project_bwd.restype = st
    lib.yoco_kv_project_bwd.argtypes = [vp, i32, i64, i32, vp, f32, vp, vp, i32, i32, i32, vp, vp, i32, vp, vp, vp,
                                        vp, vp, sz, vp]
    lib.yoco_q_project_bwd.restype = st
    lib.yoco_q_project_bwd.argtypes = [vp, i32, i64, i32, vp, f32, vp, i32, i32, i32, vp, i32, vp, vp, vp, vp, sz,
                                       vp]
    lib.yoco_gret_prefill_workspace.restype = st
    lib.yoco_gret_prefill_workspace.argtypes = [i64, i32, i32, i32, ctypes.POINTER(sz)]
    lib.yoco_gret_prefill.restype = st
    lib.yoco_gret_prefill.argtypes = [vp, vp, vp, i32, vp, f32, i64, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.yoco_gret_decode.restype = st
    lib.yoco_gret_decode.argtypes = [vp, vp, vp, i32, vp, f32, i32, i32, i32, vp, vp, vp]
    lib.yoco_cross_attn_decode_workspace.restype = st
    lib.yoco_cross_attn_decode_workspace.argtypes = [cp, i32, i64, ctypes.POINTER(sz)]
    lib.yoco_cross_attn_decode.restype = st
    lib.yoco_cross_attn_decode.argtypes = [vp, i32, i32, cp, f32, vp, vp, vp, sz, i64, vp]
    lib.yoco_cross_attn_decode_noalloc.restype = st
    lib.yoco_cross_attn_decode_noalloc.argtypes = [vp, i32, i32, cp, f32, vp, vp, i64, vp]
    return lib


def lib():
    """The loaded C library (raises if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m yoco_shared_kv_amd.build`; "
                    "there is no fallback path")
            _lib = _declare(ctypes.CDLL(LIB_PATH))
        return _lib


def check(status: int) -> None:
    if status != 0:
        raise YocoError(status, lib().yoco_last_error().decode("utf-8", "replace"))
