"""ctypes loader for libmccb.so. Fails loudly: there is no fallback path."""
from __future__ import annotations

import ctypes
import os

from . import build as _build

_lib = None


class MccbError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class Plan(ctypes.Structure):
    _fields_ = [("rows_per_turn", ctypes.c_int64), ("rows_per_round", ctypes.c_int64),
                ("rows_per_strip", ctypes.c_int64),
                ("n_strips", ctypes.c_int64), ("cols_per_block", ctypes.c_int64),
                ("n_col_blocks", ctypes.c_int64), ("waves_per_block", ctypes.c_int64),
                ("workspace_size", ctypes.c_uint64),
                ("fwd_rows_per_tile", ctypes.c_int64), ("fwd_cols_per_tile", ctypes.c_int64),
                ("fwd_n_col_tiles", ctypes.c_int64), ("fwd_n_row_tiles", ctypes.c_int64),
                ("group_spacing", ctypes.c_int64)]


class Strides(ctypes.Structure):
    """mccb_strides_t: element strides of gradY / x (S, B, H), weight (k, H), mask (B, S)."""
    _fields_ = [("gradY", ctypes.c_int64 * 3), ("x", ctypes.c_int64 * 3),
                ("weight", ctypes.c_int64 * 2), ("mask", ctypes.c_int64 * 2)]


def lib() -> ctypes.CDLL:
    """The loaded library, building it first if no build exists."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            if os.environ.get("MCCB_LIBRARY"):
                raise OSError(f"MCCB_LIBRARY={_build.LIB} does not exist")
            _build.build_library()
        L = ctypes.CDLL(_build.LIB)
        i64, u64, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
        L.mccb_get_workspace_size.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(u64)]
        L.mccb_get_workspace_size.restype = ctypes.c_int
        L.mccb_get_plan.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.POINTER(Plan)]
        L.mccb_get_plan.restype = ctypes.c_int
        L.mccb_backward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int,
                                    vp, u64, vp]
        L.mccb_backward.restype = ctypes.c_int
        L.mccb_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int,
                                            vp]
        L.mccb_backward_noalloc.restype = ctypes.c_int
        L.mccb_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp]
        L.mccb_forward.restype = ctypes.c_int
        sp = ctypes.POINTER(Strides)
        L.mccb_get_workspace_size_ex.argtypes = [vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, sp,
                                                 ctypes.POINTER(u64)]
        L.mccb_get_workspace_size_ex.restype = ctypes.c_int
        L.mccb_backward_ex.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                       sp, vp, u64, vp]
        L.mccb_backward_ex.restype = ctypes.c_int
        L.mccb_forward_get_workspace_size_ex.argtypes = [vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                                         sp, ctypes.POINTER(u64)]
        L.mccb_forward_get_workspace_size_ex.restype = ctypes.c_int
        L.mccb_forward_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, sp, vp, u64,
                                      vp]
        L.mccb_forward_ex.restype = ctypes.c_int
        L.mccb_varlen_get_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int,
                                                     ctypes.POINTER(u64)]
        L.mccb_varlen_get_workspace_size.restype = ctypes.c_int
        L.mccb_varlen_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                           ctypes.c_int, vp, u64, vp]
        L.mccb_varlen_backward.restype = ctypes.c_int
        L.mccb_varlen_forward_get_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int,
                                                             ctypes.POINTER(u64)]
        L.mccb_varlen_forward_get_workspace_size.restype = ctypes.c_int
        L.mccb_varlen_forward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, vp,
                                          u64, vp]
        L.mccb_varlen_forward.restype = ctypes.c_int
        L.mccb_status_string.argtypes = [ctypes.c_int]
        L.mccb_status_string.restype = ctypes.c_char_p
        L.mccb_profile_begin.argtypes = [ctypes.c_int]
        L.mccb_profile_begin.restype = ctypes.c_int
        L.mccb_profile_end.argtypes = [ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int)]
        L.mccb_profile_end.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mccb_status_string(int(status)).decode()
