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
        u8p = ctypes.POINTER(ctypes.c_uint8)
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.orc_compact_flags_b32.argtypes = [u32p, u8p, u32p, i64]
        L.orc_compact_flags_b32.restype = i64
        L.orc_select_flags.argtypes = [u8p, i32p, i64]
        L.orc_select_flags.restype = i64
        L.orc_compact_kv_i32.argtypes = [i32p, u32p, i32p, u32p, i64, c_int, i32, i32]
        L.orc_compact_kv_i32.restype = i64
        L.orc_compact_kv_f32.argtypes = [f32p, u32p, f32p, u32p, i64, c_int, f32, f32]
        L.orc_compact_kv_f32.restype = i64
        L.orc_pred_args_ok_i64.argtypes = [c_int, i32]
        L.orc_pred_args_ok_i64.restype = c_int
        L.orc_pred_i64.argtypes = [i64, c_int, i32]
        L.orc_pred_i64.restype = c_int
        L.orc_compact_i64.argtypes = [i64p, i64p, i64, c_int, i32]
        L.orc_compact_i64.restype = i64
        L.orc_select_index_i64.argtypes = [i64p, i32p, i64, c_int, i32]
        L.orc_select_index_i64.restype = i64
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


def _b32(a) -> np.ndarray:
    """32-bit words of an int32, uint32 or float32 array (bits unchanged)."""
    a = np.ascontiguousarray(a)
    assert a.dtype.itemsize == 4, a.dtype
    return a.view(np.uint32)


def _flag_bytes(f) -> np.ndarray:
    f = np.ascontiguousarray(f)
    assert f.dtype.itemsize == 1, f.dtype
    return f.view(np.uint8)


def compact_flags(x, f):
    """(survivors, count): the 32-bit elements of x whose flag byte is nonzero,
    in input order, with x's dtype."""
    x = np.ascontiguousarray(x)
    w = _b32(x)
    fb = _flag_bytes(f)
    assert fb.size == w.size
    out = np.empty(w.size, np.uint32)
    m = lib().orc_compact_flags_b32(_ptr(w, ctypes.c_uint32), _ptr(fb, ctypes.c_uint8),
                                    _ptr(out, ctypes.c_uint32), w.size)
    return out[:m].view(x.dtype).copy(), int(m)


def select_flags(f):
    """(indices, count): positions whose flag byte is nonzero."""
    fb = _flag_bytes(f)
    idx = np.empty(fb.size, np.int32)
    m = lib().orc_select_flags(_ptr(fb, ctypes.c_uint8), _ptr(idx, ctypes.c_int32), fb.size)
    return idx[:m].copy(), int(m)


def compact_kv(keys, vals, pred: int, a=0, b=0):
    """(keys_out, vals_out, count): the pairs whose key satisfies the predicate,
    in input order. int32 keys take the integer predicates, float32 keys the
    fp32 ones; values are any 32-bit type, moved bit for bit."""
    keys = np.ascontiguousarray(keys)
    vals = np.ascontiguousarray(vals)
    vw = _b32(vals)
    assert keys.size == vw.size
    ok = np.empty(keys.size, keys.dtype)
    ov = np.empty(vw.size, np.uint32)
    if keys.dtype == np.int32:
        m = lib().orc_compact_kv_i32(_ptr(keys, ctypes.c_int32), _ptr(vw, ctypes.c_uint32),
                                     _ptr(ok, ctypes.c_int32), _ptr(ov, ctypes.c_uint32),
                                     keys.size, pred, int(a), int(b))
    elif keys.dtype == np.float32:
        m = lib().orc_compact_kv_f32(_ptr(keys, ctypes.c_float), _ptr(vw, ctypes.c_uint32),
                                     _ptr(ok, ctypes.c_float), _ptr(ov, ctypes.c_uint32),
                                     keys.size, pred, float(a), float(b))
    else:
        raise TypeError(keys.dtype)
    return ok[:m].copy(), ov[:m].view(vals.dtype).copy(), int(m)


def _i64(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint64:
        return a.view(np.int64)
    if a.dtype != np.int64:
        a = a.astype(np.int64)
    return a


def pred_args_ok_i64(pred: int, pa: int = 0) -> bool:
    return bool(lib().orc_pred_args_ok_i64(pred, pa))


def pred_i64(x: int, pred: int, pa: int = 0) -> int:
    """P(x) for one 64-bit value (given as a Python int in int64 or uint64 range)."""
    return int(lib().orc_pred_i64(int(np.array(x, dtype=np.uint64 if x >= 2**63 else np.int64)
                                      .view(np.int64)), pred, pa))


def compact_i64(x, pred: int, pa: int = 0):
    """(survivors, count) of 64-bit elements in input order."""
    x = _i64(x)
    out = np.empty(x.size, np.int64)
    m = lib().orc_compact_i64(_ptr(x, ctypes.c_int64), _ptr(out, ctypes.c_int64), x.size,
                              pred, pa)
    return out[:m].copy(), int(m)


def select_index_i64(x, pred: int, pa: int = 0):
    """(indices, count) of the 64-bit elements for which the predicate holds."""
    x = _i64(x)
    idx = np.empty(x.size, np.int32)
    m = lib().orc_select_index_i64(_ptr(x, ctypes.c_int64), _ptr(idx, ctypes.c_int32), x.size,
                                   pred, pa)
    return idx[:m].copy(), int(m)
