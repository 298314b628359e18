"""Sequential CPU oracle (test infrastructure only).

Only the tests, the smoke check and the benchmark's cpu_baseline leg may use
this package. The product path never imports it. It wraps ``oracle.c`` (plain
C, built with gcc) through ctypes and works on numpy arrays on the host.

What each function computes, and which passage of the pages it follows, is
stated in ``oracle.c``. Every function is pinned against fixed facts (printed
transcripts, closed forms, invariants, brute force) in
``tests/test_oracle_pins.py``; none is parity unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Predicate numbering as the oracle defines it (checked against the C ABI).
PRED_NONZERO, PRED_ODD, PRED_EVEN, PRED_BIT_SET, PRED_BIT_CLEAR, PRED_MOD_LT = range(6)
PRED_F32_NONZERO, PRED_F32_GT, PRED_F32_LT, PRED_F32_IN = range(6, 10)

_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, sequential, no OpenMP)."""
    tmp = _LIB + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC",
         _SRC, "-o", tmp],
        check=True,
    )
    os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        i32p = ctypes.POINTER(ctypes.c_int32)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64, i32, c_int = ctypes.c_int64, ctypes.c_int32, ctypes.c_int
        L.orc_pred_id.argtypes = [c_int]
        L.orc_pred_id.restype = c_int
        L.orc_pred_args_ok.argtypes = [c_int, i32, i32]
        L.orc_pred_args_ok.restype = c_int
        L.orc_pred.argtypes = [i32, c_int, i32, i32]
        L.orc_pred.restype = c_int
        L.orc_flags.argtypes = [i32p, i32p, i64, c_int, i32, i32]
        L.orc_flags.restype = None
        L.orc_exclusive_scan_i32.argtypes = [i32p, i32p, i64, i32p]
        L.orc_exclusive_scan_i32.restype = None
        L.orc_exclusive_scan_f32.argtypes = [f32p, f64p, i64, f64p]
        L.orc_exclusive_scan_f32.restype = None
        L.orc_inclusive_scan_i32.argtypes = [i32p, i32p, i64]
        L.orc_inclusive_scan_i32.restype = None
        L.orc_inclusive_scan_f32.argtypes = [f32p, f64p, i64]
        L.orc_inclusive_scan_f32.restype = None
        L.orc_select_index_i32.argtypes = [i32p, i32p, i64, c_int, i32, i32]
        L.orc_select_index_i32.restype = i64
        f32 = ctypes.c_float
        L.orc_pred_f32.argtypes = [f32, c_int, f32, f32]
        L.orc_pred_f32.restype = c_int
        L.orc_compact_f32.argtypes = [f32p, f32p, i64, c_int, f32, f32]
        L.orc_compact_f32.restype = i64
        L.orc_partition_f32.argtypes = [f32p, f32p, i64, c_int, f32, f32]
        L.orc_partition_f32.restype = i64
        L.orc_select_index_f32.argtypes = [f32p, i32p, i64, c_int, f32, f32]
        L.orc_select_index_f32.restype = i64
        L.orc_count.argtypes = [i32p, i64, c_int, i32, i32]
        L.orc_count.restype = i64
        L.orc_compact_i32.argtypes = [i32p, i32p, i64, c_int, i32, i32, i32p]
        L.orc_compact_i32.restype = i64
        L.orc_partition_i32.argtypes = [i32p, i32p, i64, c_int, i32, i32]
        L.orc_partition_i32.restype = i64
        L.orc_radix_sort_u32.argtypes = [u32p, u32p, u32p, i64, c_int]
        L.orc_radix_sort_u32.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _i32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.int32:
        a = a.astype(np.int32)
    return a


def pred_args_ok(pred: int, pa: int = 0, pb: int = 0) -> bool:
    return bool(lib().orc_pred_args_ok(pred, pa, pb))


def pred(x: int, pred: int, pa: int = 0, pb: int = 0) -> int:
    """P(x) for one int32 value."""
    return int(lib().orc_pred(int(np.int32(x)), pred, pa, pb))


def flags(x, pred: int, pa: int = 0, pb: int = 0) -> np.ndarray:
    x = _i32(x)
    f = np.empty(x.size, np.int32)
    lib().orc_flags(_ptr(x, ctypes.c_int32), _ptr(f, ctypes.c_int32), x.size, pred, pa, pb)
    return f


def exclusive_scan_i32(x):
    """(out, total): exclusive scan with modulo-2^32 wrap."""
    x = _i32(x)
    out = np.empty(x.size, np.int32)
    total = ctypes.c_int32(0)
    lib().orc_exclusive_scan_i32(_ptr(x, ctypes.c_int32), _ptr(out, ctypes.c_int32), x.size,
                                 ctypes.byref(total))
    return out, int(total.value)


def exclusive_scan_f32(x):
    """(out_f64, total_f64): exclusive scan of fp32 values accumulated in fp64."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, np.float64)
    total = ctypes.c_double(0.0)
    lib().orc_exclusive_scan_f32(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_double), x.size,
                                 ctypes.byref(total))
    return out, float(total.value)


def inclusive_scan_i32(x) -> np.ndarray:
    """out[i] = x[0] + ... + x[i] with modulo-2^32 wrap."""
    x = _i32(x)
    out = np.empty(x.size, np.int32)
    lib().orc_inclusive_scan_i32(_ptr(x, ctypes.c_int32), _ptr(out, ctypes.c_int32), x.size)
    return out


def inclusive_scan_f32(x) -> np.ndarray:
    """out[i] = x[0] + ... + x[i] of fp32 values, accumulated and returned in fp64."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.size, np.float64)
    lib().orc_inclusive_scan_f32(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_double), x.size)
    return out


def select_index_i32(x, pred: int, pa: int = 0, pb: int = 0):
    """(indices, count): positions of the elements for which the predicate holds."""
    x = _i32(x)
    idx = np.empty(x.size, np.int32)
    m = lib().orc_select_index_i32(_ptr(x, ctypes.c_int32), _ptr(idx, ctypes.c_int32), x.size,
                                   pred, pa, pb)
    return idx[:m].copy(), int(m)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def pred_f32(x: float, pred: int, a: float = 0.0, b: float = 0.0) -> int:
    """P(x) for one fp32 value."""
    return int(lib().orc_pred_f32(float(np.float32(x)), pred, a, b))


def compact_f32(x, pred: int, a: float = 0.0, b: float = 0.0):
    """(survivors, count) of fp32 values in input order."""
    x = _f32(x)
    out = np.empty(x.size, np.float32)
    m = lib().orc_compact_f32(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_float), x.size, pred, a, b)
    return out[:m].copy(), int(m)


def partition_f32(x, pred: int, a: float = 0.0, b: float = 0.0):
    """(out, kept): predicate-true fp32 values first, both halves in input order."""
    x = _f32(x)
    out = np.empty(x.size, np.float32)
    k = lib().orc_partition_f32(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_float), x.size, pred, a, b)
    return out, int(k)


def select_index_f32(x, pred: int, a: float = 0.0, b: float = 0.0):
    """(indices, count) of the fp32 values for which the predicate holds."""
    x = _f32(x)
    idx = np.empty(x.size, np.int32)
    m = lib().orc_select_index_f32(_ptr(x, ctypes.c_float), _ptr(idx, ctypes.c_int32), x.size,
                                   pred, a, b)
    return idx[:m].copy(), int(m)


def count(x, pred: int, pa: int = 0, pb: int = 0) -> int:
    x = _i32(x)
    return int(lib().orc_count(_ptr(x, ctypes.c_int32), x.size, pred, pa, pb))


def compact_i32(x, pred: int, pa: int = 0, pb: int = 0, want_ranks: bool = False):
    """(survivors, count[, ranks]) in input order."""
    x = _i32(x)
    out = np.empty(x.size, np.int32)
    ranks = np.empty(x.size, np.int32) if want_ranks else None
    m = lib().orc_compact_i32(_ptr(x, ctypes.c_int32), _ptr(out, ctypes.c_int32), x.size,
                              pred, pa, pb,
                              _ptr(ranks, ctypes.c_int32) if want_ranks else None)
    if want_ranks:
        return out[:m].copy(), int(m), ranks
    return out[:m].copy(), int(m)


def partition_i32(x, pred: int, pa: int = 0, pb: int = 0):
    """(out, kept): predicate-true elements first, both halves in input order."""
    x = _i32(x)
    out = np.empty(x.size, np.int32)
    k = lib().orc_partition_i32(_ptr(x, ctypes.c_int32), _ptr(out, ctypes.c_int32), x.size,
                                pred, pa, pb)
    return out, int(k)


def radix_sort_u32(x, passes: int = 32) -> np.ndarray:
    """LSB-first chained stable 1-bit partitions (bit-clear first)."""
    x = np.ascontiguousarray(x, dtype=np.uint32)
    out = np.empty_like(x)
    tmp = np.empty_like(x)
    lib().orc_radix_sort_u32(_ptr(x, ctypes.c_uint32), _ptr(out, ctypes.c_uint32),
                             _ptr(tmp, ctypes.c_uint32), x.size, passes)
    return out
