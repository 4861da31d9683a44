"""CPU fp64 oracle for the masked causal depthwise conv1d backward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never calls it and shares no code with it.

The arithmetic lives in ``mccb_oracle.c`` (plain C loops in fp64, written from the equations of the
"aclnnMaskedCausalConv1dBackward" page, section 功能说明 / function description). This module only
marshals numpy arrays into it.

Every function here is pinned by ``tests/test_oracle.py`` (hand-worked cases, the page's call
example, PyTorch CPU autograd, the adjoint identity, invariants, an exhaustive codec check).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mccb_oracle.c")
# MCCB_ORACLE_LIBRARY names another build of the oracle to load by default (the tests'
# sanitized build).
_LIB = os.environ.get("MCCB_ORACLE_LIBRARY") or os.path.join(_HERE, "libmccb_oracle.so")

DTYPE_CODE = {"bf16": 0, "fp16": 1}

# Compiler line: -ffp-contract=off keeps every a*b + c as a rounded product followed by a rounded
# sum, exactly as the C source reads.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-std=c11"]


def build(src: str = _SRC, out: str = _LIB, extra: list[str] | None = None) -> str:
    """Compile the oracle with gcc. Returns the path of the shared library."""
    cmd = ["gcc", *CFLAGS, *(extra or []), src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f64p = ctypes.POINTER(ctypes.c_double)


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    i64 = ctypes.c_int64
    lib.oracle_decode.argtypes = [ctypes.c_int, _u16p, _f64p, i64]
    lib.oracle_decode.restype = None
    lib.oracle_encode.argtypes = [ctypes.c_int, _f64p, _u16p, i64]
    lib.oracle_encode.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    lib.oracle_backward.argtypes = [ctypes.c_int, i64, i64, i64, _u16p, _u16p, _u16p, _u8p,
                                    _f64p, _u16p, _f64p, _f64p, _u16p]
    lib.oracle_backward.restype = ctypes.c_int
    lib.oracle_forward.argtypes = [i64, i64, i64, _f64p, _f64p, _u8p, _f64p]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_backward_w.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, _u16p, _u16p,
                                      _u16p, _u8p, _f64p, _u16p, _f64p, _f64p, _u16p]
    lib.oracle_backward_w.restype = ctypes.c_int
    lib.oracle_forward_w.argtypes = [ctypes.c_int, i64, i64, i64, _f64p, _f64p, _u8p, _f64p]
    lib.oracle_forward_w.restype = ctypes.c_int
    lib.oracle_backward_rows_w.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, i64, i64,
                                           _u16p, _u16p, _u16p, _u8p, _u16p, _f64p, _f64p]
    lib.oracle_backward_rows_w.restype = ctypes.c_int
    _i64p = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_backward_varlen.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, _i64p, _u16p,
                                           _u16p, _u16p, _u8p, _f64p, _u16p, _f64p, _f64p, _u16p]
    lib.oracle_backward_varlen.restype = ctypes.c_int
    lib.oracle_forward_varlen.argtypes = [ctypes.c_int, i64, i64, i64, _i64p, _f64p, _f64p, _u8p,
                                          _f64p]
    lib.oracle_forward_varlen.restype = ctypes.c_int
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load a compiled oracle library (building the default one if it is not there yet)."""
    if path is None:
        path = _LIB
        if not os.path.exists(path):
            build()
    return _bind(ctypes.CDLL(path))


class Oracle:
    """Thin numpy front end over one compiled oracle library."""

    def __init__(self, path: str | None = None):
        self.lib = load(path)

    # -- codec ------------------------------------------------------------------------------------
    def decode(self, dtype: str, bits: np.ndarray) -> np.ndarray:
        b = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.oracle_decode(DTYPE_CODE[dtype], _ptr(b, _u16p), _ptr(out, _f64p), b.size)
        return out

    def encode(self, dtype: str, values: np.ndarray) -> np.ndarray:
        v = np.ascontiguousarray(values, dtype=np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.oracle_encode(DTYPE_CODE[dtype], _ptr(v, _f64p), _ptr(out, _u16p), v.size)
        return out

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        """OpenMP threads of the following calls (timing only: results do not depend on it)."""
        self.lib.oracle_set_num_threads(int(n))

    # -- the backward -----------------------------------------------------------------------------
    def backward(self, dtype: str, gY: np.ndarray, x: np.ndarray, w: np.ndarray,
                 mask: np.ndarray | None, want_gx64: bool = True) -> dict:
        """gY, x: uint16 [S,B,H]; w: uint16 [W,H] (the window W is w's first dimension, 3 on the
        page); mask: uint8/bool [B,S] or None.

        Returns a dict with ``gx16`` (uint16 [S,B,H]), ``gx64`` (float64 [S,B,H], if asked),
        ``gw16`` (uint16 [W,H]), ``gw64`` (float64 [W,H]) and ``gwrss`` (float64 [W,H]).
        """
        gY = np.ascontiguousarray(gY, dtype=np.uint16)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        if gY.ndim != 3 or x.shape != gY.shape:
            raise ValueError("gY and x must both be [S,B,H]")
        S, B, H = gY.shape
        if w.ndim != 2 or w.shape[1] != H or w.shape[0] < 1:
            raise ValueError("w must be [W,H]")
        W = int(w.shape[0])
        m = None
        if mask is not None:
            m = np.ascontiguousarray(mask).astype(np.uint8, copy=False)
            if m.shape != (B, S):
                raise ValueError("mask must be [B,S]")
        out = {
            "gx16": np.empty((S, B, H), dtype=np.uint16),
            "gw16": np.empty((W, H), dtype=np.uint16),
            "gw64": np.empty((W, H), dtype=np.float64),
            "gwrss": np.empty((W, H), dtype=np.float64),
        }
        if want_gx64:
            out["gx64"] = np.empty((S, B, H), dtype=np.float64)
        rc = self.lib.oracle_backward_w(
            DTYPE_CODE[dtype], W, S, B, H, _ptr(gY, _u16p), _ptr(x, _u16p), _ptr(w, _u16p),
            None if m is None else _ptr(m, _u8p),
            _ptr(out["gx64"], _f64p) if want_gx64 else None, _ptr(out["gx16"], _u16p),
            _ptr(out["gw64"], _f64p), _ptr(out["gwrss"], _f64p), _ptr(out["gw16"], _u16p))
        if rc != 0:
            raise RuntimeError(f"oracle_backward failed ({rc})")
        return out

    def backward_rows(self, dtype: str, S: int, r0: int, r1: int, gY_rows: np.ndarray,
                      x_rows: np.ndarray, w: np.ndarray, mask: np.ndarray | None,
                      gw_acc: np.ndarray, gw_sq: np.ndarray | None = None) -> np.ndarray:
        """Rows r0 .. r1-1 of a problem with S rows: returns gradX of those rows (uint16
        [r1-r0,B,H]) and adds their gradWeight terms (and squared terms) into the float64 [W,H]
        arrays gw_acc (and gw_sq). gY_rows holds gradY rows r0 .. min(r1+W-1, S)-1, x_rows x rows
        r0 .. r1-1, mask is the whole [B,S] mask or None."""
        gY_rows = np.ascontiguousarray(gY_rows, dtype=np.uint16)
        x_rows = np.ascontiguousarray(x_rows, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        W = int(w.shape[0])
        n, B, H = x_rows.shape
        if n != r1 - r0 or gY_rows.shape != (min(r1 + W - 1, S) - r0, B, H):
            raise ValueError("row slabs do not match r0, r1, S and W")
        if gw_acc.dtype != np.float64 or gw_acc.shape != (W, H) or not gw_acc.flags.c_contiguous:
            raise ValueError("gw_acc must be a contiguous float64 [W,H] array")
        if gw_sq is not None and (gw_sq.dtype != np.float64 or gw_sq.shape != (W, H) or
                                  not gw_sq.flags.c_contiguous):
            raise ValueError("gw_sq must be a contiguous float64 [W,H] array")
        m = None
        if mask is not None:
            m = np.ascontiguousarray(mask).astype(np.uint8, copy=False)
            if m.shape != (B, S):
                raise ValueError("mask must be the whole [B,S] mask")
        gx16 = np.empty((n, B, H), dtype=np.uint16)
        rc = self.lib.oracle_backward_rows_w(
            DTYPE_CODE[dtype], W, S, B, H, r0, r1, _ptr(gY_rows, _u16p), _ptr(x_rows, _u16p),
            _ptr(w, _u16p), None if m is None else _ptr(m, _u8p), _ptr(gx16, _u16p),
            _ptr(gw_acc, _f64p), None if gw_sq is None else _ptr(gw_sq, _f64p))
        if rc != 0:
            raise RuntimeError(f"oracle_backward_rows_w failed ({rc})")
        return gx16

    def forward(self, x64: np.ndarray, w64: np.ndarray, mask: np.ndarray | None) -> np.ndarray:
        """fp64 causal depthwise forward y = mask * conv(x, w), w [W,H]; used by the adjoint test
        and, rounded by forward16, as the forward's reference."""
        x64 = np.ascontiguousarray(x64, dtype=np.float64)
        w64 = np.ascontiguousarray(w64, dtype=np.float64)
        S, B, H = x64.shape
        if w64.ndim != 2 or w64.shape[1] != H or w64.shape[0] < 1:
            raise ValueError("w must be [W,H]")
        m = None if mask is None else np.ascontiguousarray(mask).astype(np.uint8, copy=False)
        y = np.empty_like(x64)
        rc = self.lib.oracle_forward_w(int(w64.shape[0]), S, B, H, _ptr(x64, _f64p),
                                       _ptr(w64, _f64p), None if m is None else _ptr(m, _u8p),
                                       _ptr(y, _f64p))
        if rc != 0:
            raise RuntimeError(f"oracle_forward failed ({rc})")
        return y


    def forward16(self, dtype: str, x16: np.ndarray, w16: np.ndarray,
                  mask: np.ndarray | None) -> dict:
        """The forward on 16-bit inputs: decode exactly, compute in fp64, round once to `dtype`
        with the oracle's own encoder. Returns {"y64": fp64 values, "y16": rounded bit patterns}."""
        x64 = self.decode(dtype, np.ascontiguousarray(x16, dtype=np.uint16))
        w64 = self.decode(dtype, np.ascontiguousarray(w16, dtype=np.uint16))
        y64 = self.forward(x64, w64, mask)
        return {"y64": y64, "y16": self.encode(dtype, y64)}


    # -- packed variable-length layout ------------------------------------------------------------
    def backward_varlen(self, dtype: str, gY: np.ndarray, x: np.ndarray, w: np.ndarray,
                        cu: np.ndarray, mask: np.ndarray | None, want_gx64: bool = True) -> dict:
        """gY, x: uint16 [T,H] packed tokens; w: uint16 [W,H]; cu: int64 [n] cumulative sequence
        ends (cu[-1] == T); mask: uint8/bool [T] or None. Same outputs as backward()."""
        gY = np.ascontiguousarray(gY, dtype=np.uint16)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.uint16)
        cu = np.ascontiguousarray(cu, dtype=np.int64)
        T, H = gY.shape
        W = int(w.shape[0])
        if x.shape != (T, H) or w.shape != (W, H):
            raise ValueError("gY, x must be [T,H] and w [W,H]")
        m = None if mask is None else np.ascontiguousarray(mask).astype(np.uint8, copy=False)
        out = {"gx16": np.empty((T, H), np.uint16), "gw16": np.empty((W, H), np.uint16),
               "gw64": np.empty((W, H), np.float64), "gwrss": np.empty((W, H), np.float64)}
        if want_gx64:
            out["gx64"] = np.empty((T, H), np.float64)
        rc = self.lib.oracle_backward_varlen(
            DTYPE_CODE[dtype], W, T, H, cu.size, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            _ptr(gY, _u16p), _ptr(x, _u16p), _ptr(w, _u16p), None if m is None else _ptr(m, _u8p),
            _ptr(out["gx64"], _f64p) if want_gx64 else None, _ptr(out["gx16"], _u16p),
            _ptr(out["gw64"], _f64p), _ptr(out["gwrss"], _f64p), _ptr(out["gw16"], _u16p))
        if rc != 0:
            raise RuntimeError(f"oracle_backward_varlen failed ({rc})")
        return out

    def forward_varlen(self, x64: np.ndarray, w64: np.ndarray, cu: np.ndarray,
                       mask: np.ndarray | None) -> np.ndarray:
        x64 = np.ascontiguousarray(x64, dtype=np.float64)
        w64 = np.ascontiguousarray(w64, dtype=np.float64)
        cu = np.ascontiguousarray(cu, dtype=np.int64)
        T, H = x64.shape
        m = None if mask is None else np.ascontiguousarray(mask).astype(np.uint8, copy=False)
        y = np.empty_like(x64)
        rc = self.lib.oracle_forward_varlen(
            int(w64.shape[0]), T, H, cu.size, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            _ptr(x64, _f64p), _ptr(w64, _f64p), None if m is None else _ptr(m, _u8p),
            _ptr(y, _f64p))
        if rc != 0:
            raise RuntimeError(f"oracle_forward_varlen failed ({rc})")
        return y

    def forward16_varlen(self, dtype: str, x16: np.ndarray, w16: np.ndarray, cu: np.ndarray,
                         mask: np.ndarray | None) -> dict:
        x64 = self.decode(dtype, np.ascontiguousarray(x16, dtype=np.uint16))
        w64 = self.decode(dtype, np.ascontiguousarray(w16, dtype=np.uint16))
        y64 = self.forward_varlen(x64, w64, cu, mask)
        return {"y64": y64, "y16": self.encode(dtype, y64)}


def _ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(typ)


_default: Oracle | None = None


def get() -> Oracle:
    """The process-wide oracle over the default library."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
