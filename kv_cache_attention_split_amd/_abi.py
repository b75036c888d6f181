"""ctypes declarations of libispa.so (mirrors include/ispa.h)."""
from __future__ import annotations

import ctypes
import os
import threading

ISPA_OK = 0
ISPA_E_ARG = -1
ISPA_E_UNSUPPORTED = -2
ISPA_E_WORKSPACE = -3
ISPA_E_HIP = -4
ISPA_F32 = 0
ISPA_BF16 = 1
ISPA_NOALLOC_SCRATCH_BYTES = 16 << 20   # include/ispa.h

_HERE = os.path.dirname(os.path.abspath(__file__))
_DEFAULT_LIB = os.path.join(_HERE, "libispa.so")


class IspaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class KVSegment(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("row_stride", ctypes.c_int64)]


class KVBias(ctypes.Structure):
    _fields_ = [("sink", ctypes.c_void_p), ("cur", ctypes.c_void_p), ("hist", ctypes.c_void_p),
                ("sink_head_stride", ctypes.c_int64), ("cur_head_stride", ctypes.c_int64),
                ("hist_head_stride", ctypes.c_int64)]


_lib = None
_lock = threading.Lock()

c_vp = ctypes.c_void_p
c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_f32 = ctypes.c_float
c_sz = ctypes.c_size_t
c_int = ctypes.c_int

# symbol -> (restype, argtypes); the list is the C ABI of include/ispa.h
SIGNATURES = {
    "ispa_attn_dual": (c_int, [c_int, c_i32, c_i32, c_f32, c_vp, c_i64, c_i64, KVSegment, KVSegment,
                               KVSegment, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "ispa_attn_dual_balanced_workspace": (c_sz, [c_int, c_i32, c_i32, c_i64, c_i64, c_i64]),
    "ispa_attn_dual_balanced": (c_int, [c_int, c_i32, c_i32, c_f32, c_vp, c_i64, c_i64, KVSegment, KVSegment,
                                        KVSegment, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "ispa_attn_dual_biased": (c_int, [c_int, c_i32, c_i32, c_f32, c_vp, c_i64, c_i64, KVSegment, KVSegment,
                                      KVSegment, ctypes.POINTER(KVBias), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "ispa_kv_merge": (c_int, [c_int, c_i32, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_i64,
                              c_vp, c_vp]),
    "ispa_fp8_head_scales": (c_int, [c_int, c_vp, c_i64, c_i32, c_i32, c_i64, c_vp, c_vp]),
    "ispa_fp8_quantize": (c_int, [c_int, c_vp, c_i64, c_i32, c_i32, c_i64, c_vp, c_vp, c_i64, c_vp]),
    "ispa_attn_dual_fp8": (c_int, [c_i32, c_i32, c_f32, c_vp, c_i64, c_i64, c_vp, KVSegment, KVSegment, KVSegment,
                                   c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "ispa_attn_dual_fp8_pv": (c_int, [c_i32, c_i32, c_f32, c_vp, c_i64, c_i64, c_vp, KVSegment, KVSegment,
                                      KVSegment, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "ispa_future_scores_workspace": (c_sz, [c_i32, c_i64]),
    "ispa_future_scores": (c_int, [c_int, c_i32, c_i32, c_f32, c_vp, c_i64, c_i64, KVSegment, KVSegment,
                                   KVSegment, c_vp, c_i64, c_f32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "ispa_future_scores_noalloc": (c_int, [c_int, c_i32, c_i32, c_f32, c_vp, c_i64, c_i64, KVSegment, KVSegment,
                                           KVSegment, c_vp, c_i64, c_f32, c_vp, c_vp, c_vp]),
    "ispa_absorb_accumulate_workspace": (c_sz, [c_i64, c_i32]),
    "ispa_absorb_accumulate": (c_int, [c_int, c_i64, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "ispa_absorb_accumulate_batched": (c_int, [c_int, c_i64, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "ispa_absorb_accumulate_fp8": (c_int, [c_i64, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                           c_sz, c_vp]),
    "ispa_absorb_solve_workspace": (c_sz, [c_i32, c_i32]),
    "ispa_absorb_solve": (c_int, [c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "ispa_absorb_solve_eps_workspace": (c_sz, [c_i32, c_i32]),
    "ispa_absorb_solve_eps": (c_int, [c_i32, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp,
                                      c_vp, c_sz, c_vp]),
    "ispa_layer_error_workspace": (c_sz, [c_i32, c_i32]),
    "ispa_layer_error": (c_int, [c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "ispa_rank_layers": (c_int, [c_vp, c_i32, c_i32, c_vp, c_vp]),
    "ispa_apply_delta": (c_int, [c_i32, c_i32, c_vp, c_vp, c_i32, c_vp, c_vp]),
    "ispa_project": (c_int, [c_i64, c_i32, c_i32, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp]),
    "ispa_kv_plan": (c_int, [c_i32, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]),
    "ispa_status_string": (ctypes.c_char_p, [c_int]),
    "ispa_version": (c_i32, []),
}


def lib_path() -> str:
    return os.environ.get("ISPA_LIB", _DEFAULT_LIB)


def lib() -> ctypes.CDLL:
    """Load libispa.so (once). Raises if the library has not been built: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            path = lib_path()
            if not os.path.exists(path):
                raise ImportError(f"libispa.so not found at {path}; build it with "
                                  "`python -m kv_cache_attention_split_amd.build`")
            handle = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().ispa_status_string(int(status)).decode()
