"""ctypes loader for libaah_attn.so (the C ABI declared in include/aah_attn.h).

The library is loaded on first use.  There is no fallback: if the shared
library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libaah_attn.so")

AAH_OK = 0
AAH_ERR_INVALID_ARG = 1
AAH_ERR_UNSUPPORTED = 2
AAH_ERR_WORKSPACE = 3
AAH_ERR_HIP = 4
AAH_BF16 = 0
AAH_F32 = 1
ABI_VERSION = 13

EXPORTS = (
    "aah_abi_version", "aah_status_string", "aah_last_error_detail", "aah_attn_fwd", "aah_attn_bwd",
    "aah_attn_workspace_size", "aah_attn_fwd_workspace_size", "aah_tile_shape", "aah_plan_fwd", "aah_plan_bwd",
    "aah_plan_fwd_split", "aah_plan_bwd_split", "aah_attn_bwd_split_workspace_size", "aah_window_stats",
    "aah_cache_clear", "aah_attn_bwd_dq", "aah_attn_bwd_dkdv", "aah_kv_cache_rows",
    "aah_attn_decode_workspace_size", "aah_kv_cache_fill", "aah_attn_decode", "aah_attn_fwd_diag",
    "aah_head_features_workspace_size", "aah_head_features", "aah_attn_decode_noalloc", "aah_cache_entries",
    "aah_attn_fwd_diag_workspace_size",
)


class WorkItem(ctypes.Structure):
    _fields_ = [("bh", ctypes.c_int32), ("tile", ctypes.c_int32), ("lo", ctypes.c_int32), ("hi", ctypes.c_int32)]


class AahError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name
        self.detail = detail


_lock = threading.Lock()
_lib = None

c_int, c_int32, c_int64, c_float, c_double, c_size_t, c_void_p = (
    ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_size_t, ctypes.c_void_p)
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_i64 = ctypes.POINTER(ctypes.c_int64)
P_int = ctypes.POINTER(ctypes.c_int)
P_double = ctypes.POINTER(ctypes.c_double)
P_item = ctypes.POINTER(WorkItem)


def _declare(lib):
    lib.aah_abi_version.restype = c_int
    lib.aah_abi_version.argtypes = []
    lib.aah_status_string.restype = ctypes.c_char_p
    lib.aah_status_string.argtypes = [c_int]
    lib.aah_last_error_detail.restype = ctypes.c_char_p
    lib.aah_last_error_detail.argtypes = []
    lib.aah_attn_fwd.restype = c_int
    lib.aah_attn_fwd.argtypes = [c_void_p, c_void_p, c_void_p, P_i32, P_i32, c_int, c_int, c_int, c_int, c_int,
                                 c_int, c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.aah_attn_fwd_diag.restype = c_int
    lib.aah_attn_fwd_diag.argtypes = [c_void_p, c_void_p, c_void_p, P_i32, P_i32, c_int, c_int, c_int, c_int, c_int,
                                      c_int, c_float, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                      c_void_p]
    lib.aah_head_features_workspace_size.restype = c_size_t
    lib.aah_head_features_workspace_size.argtypes = [c_int, c_int, c_int, c_int]
    lib.aah_head_features.restype = c_int
    lib.aah_head_features.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, P_i32, c_int, c_int, c_int,
                                      c_int, c_int, c_int, c_float, c_int, c_void_p, c_void_p, c_void_p, c_size_t,
                                      c_void_p]
    lib.aah_attn_bwd.restype = c_int
    lib.aah_attn_bwd.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, P_i32, P_i32, c_int,
                                 c_int, c_int, c_int, c_int, c_int, c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_size_t, c_void_p]
    lib.aah_attn_bwd_dkdv.restype = c_int
    lib.aah_attn_bwd_dkdv.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, P_i32, P_i32, c_int, c_int, c_int,
                                      c_int, c_int, c_int, c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.aah_attn_bwd_dq.restype = c_int
    lib.aah_attn_bwd_dq.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, P_i32, P_i32, c_int,
                                    c_int, c_int, c_int, c_int, c_int, c_float, c_void_p, c_void_p, c_size_t,
                                    c_void_p]
    lib.aah_attn_bwd_split_workspace_size.restype = c_size_t
    lib.aah_attn_bwd_split_workspace_size.argtypes = [P_i32, P_i32, c_int, c_int, c_int, c_int, c_int, c_int]
    for name in ("aah_attn_fwd_workspace_size", "aah_attn_fwd_diag_workspace_size"):
        getattr(lib, name).restype = c_size_t
        getattr(lib, name).argtypes = [P_i32, P_i32, c_int, c_int, c_int, c_int, c_int, c_int]
    lib.aah_attn_workspace_size.restype = c_size_t
    lib.aah_attn_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int]
    lib.aah_tile_shape.restype = c_int
    lib.aah_tile_shape.argtypes = [c_int, c_int, c_int, P_int, P_int]
    for name in ("aah_plan_fwd", "aah_plan_bwd"):
        fn = getattr(lib, name)
        fn.restype = c_int
        fn.argtypes = [P_i32, P_i32, c_int, c_int, c_int, c_int, c_int, c_int, c_int, P_item, c_int64, P_i64]
    for name in ("aah_plan_fwd_split", "aah_plan_bwd_split"):
        fn = getattr(lib, name)
        fn.restype = c_int
        fn.argtypes = [P_i32, P_i32, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, P_item, P_i32, c_int64,
                       P_i64, P_item, c_int64, P_i64]
    lib.aah_window_stats.restype = c_int
    lib.aah_window_stats.argtypes = [P_i32, P_i32, c_int, c_int, P_i64, P_double]
    lib.aah_cache_clear.restype = None
    lib.aah_cache_clear.argtypes = []
    lib.aah_cache_entries.restype = c_int64
    lib.aah_cache_entries.argtypes = []
    lib.aah_kv_cache_rows.restype = c_int64
    lib.aah_kv_cache_rows.argtypes = [P_i32, P_i32, c_int, c_int, c_int]
    lib.aah_attn_decode_workspace_size.restype = c_size_t
    lib.aah_attn_decode_workspace_size.argtypes = [P_i32, P_i32, c_int, c_int, c_int, c_int, c_int, c_int]
    lib.aah_kv_cache_fill.restype = c_int
    lib.aah_kv_cache_fill.argtypes = [c_void_p, c_void_p, P_i32, P_i32, c_int, c_int, c_int, c_int, c_int, c_int,
                                      c_int, c_void_p, c_void_p, c_void_p]
    lib.aah_attn_decode_noalloc.restype = c_int
    lib.aah_attn_decode_noalloc.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, P_i32, P_i32,
                                            c_int, c_int, c_int, c_int, c_int, c_int, c_float, c_void_p, c_void_p,
                                            c_void_p]
    lib.aah_attn_decode.restype = c_int
    lib.aah_attn_decode.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, P_i32, P_i32, c_int,
                                    c_int, c_int, c_int, c_int, c_int, c_float, c_void_p, c_void_p, c_void_p, c_size_t,
                                    c_void_p]


def lib():
    """The loaded library (loads it on first call)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m head_causal_local_amd.build` "
                    "(there is no fallback implementation)")
            handle = ctypes.CDLL(LIB_PATH)
            _declare(handle)
            if handle.aah_abi_version() != ABI_VERSION:
                raise RuntimeError(f"ABI version mismatch: library {handle.aah_abi_version()}, binding {ABI_VERSION}")
            _lib = handle
    return _lib


def check(status: int) -> None:
    if status != AAH_OK:
        h = lib()
        raise AahError(status, h.aah_status_string(status).decode(), h.aah_last_error_detail().decode())
