"""MI355X-native single-pass scan, stream compaction and stable partition.

A thin ctypes binding over ``libssc.so`` (the C ABI in ``include/ssc.h``).
This module only marshals arguments: every step of the computation runs in
the library's HIP kernels. PyTorch provides device memory and the current
stream. There is no CPU fallback: if the library is missing or the device is
not a gfx950 GPU, the calls raise.

Names follow the pages' vocabulary: predicate flags, exclusive scan, rank,
count (the top of the scan), compact, partition.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssc.so")
PERTURB_LIB_PATH = os.path.join(_PKG, "libssc_perturb.so")  # race-test build
STRESS_LIB_PATH = os.path.join(_PKG, "libssc_stress.so")    # race-test build, 3840-element tiles

PRED = {"nonzero": 0, "odd": 1, "even": 2, "bit_set": 3, "bit_clear": 4, "mod_lt": 5,
        "f32_nonzero": 6, "f32_gt": 7, "f32_lt": 8, "f32_in": 9}
STATUS = {0: "SSC_OK", 1: "SSC_ERR_ARG", 2: "SSC_ERR_SIZE", 3: "SSC_ERR_ALIAS",
          4: "SSC_ERR_SCRATCH", 5: "SSC_ERR_HIP", 6: "SSC_ERR_DEVICE"}

# Every symbol include/ssc.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_INT = ctypes.c_int
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float
SIGNATURES = {
    "ssc_tile_elems": (_I64, []),
    "ssc_scratch_bytes": (_SZ, [_I64]),
    "ssc_radix_sort_scratch_bytes": (_SZ, [_I64]),
    "ssc_scratch_init": (_INT, [_P, _SZ, _P]),
    "ssc_exclusive_scan_i32": (_INT, [_P, _P, _I64, _P, _P, _SZ, _P]),
    "ssc_exclusive_scan_f32": (_INT, [_P, _P, _I64, _P, _P, _SZ, _P]),
    "ssc_inclusive_scan_i32": (_INT, [_P, _P, _I64, _P, _P, _SZ, _P]),
    "ssc_inclusive_scan_f32": (_INT, [_P, _P, _I64, _P, _P, _SZ, _P]),
    "ssc_select_index_i32": (_INT, [_P, _P, _I64, _INT, _I32, _I32, _P, _P, _SZ, _P]),
    "ssc_compact_f32": (_INT, [_P, _P, _I64, _INT, _F32, _F32, _P, _P, _P, _SZ, _P]),
    "ssc_select_index_f32": (_INT, [_P, _P, _I64, _INT, _F32, _F32, _P, _P, _SZ, _P]),
    "ssc_partition_f32": (_INT, [_P, _P, _I64, _INT, _F32, _F32, _P, _P, _SZ, _P]),
    "ssc_compact_i32": (_INT, [_P, _P, _I64, _INT, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "ssc_compact_i32_noalloc": (_INT, [_P, _P, _I64, _INT, _I32, _I32, _P, _P, _P]),
    "ssc_partition_i32": (_INT, [_P, _P, _I64, _INT, _I32, _I32, _P, _P, _SZ, _P]),
    "ssc_count_if_i32": (_INT, [_P, _I64, _INT, _I32, _I32, _P, _P, _SZ, _P]),
    "ssc_compact_atomic_i32": (_INT, [_P, _P, _I64, _INT, _I32, _I32, _P, _INT, _P]),
    "ssc_radix_sort_u32": (_INT, [_P, _P, _P, _I64, _P, _SZ, _P]),
    "ssc_radix_sort4_scratch_bytes": (_SZ, [_I64]),
    "ssc_radix_sort4_u32": (_INT, [_P, _P, _P, _I64, _INT, _P, _SZ, _P]),
    "ssc_multipass_scratch_bytes": (_SZ, [_I64]),
    "ssc_exclusive_scan_multipass_i32": (_INT, [_P, _P, _I64, _P, _P, _SZ, _P]),
    "ssc_compact_multipass_i32": (_INT, [_P, _P, _I64, _INT, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "ssc_copy_i32": (_INT, [_P, _P, _I64, _P]),
    "ssc_scratch_timed_out": (_INT, [_P, _SZ, _P, _P]),
    "ssc_mark_i32": (_INT, [_P, _P, _I64, _INT, _I32, _I32, _P]),
    "ssc_scatter_i32": (_INT, [_P, _P, _P, _I64, _INT, _I32, _I32, _P, _P]),
    "ssc_compact_flags_b32": (_INT, [_P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "ssc_select_flags": (_INT, [_P, _P, _I64, _P, _P, _SZ, _P]),
    "ssc_compact_kv_i32": (_INT, [_P, _P, _P, _P, _I64, _INT, _I32, _I32, _P, _P, _SZ, _P]),
    "ssc_compact_kv_f32": (_INT, [_P, _P, _P, _P, _I64, _INT, _F32, _F32, _P, _P, _SZ, _P]),
    "ssc_compact_i64": (_INT, [_P, _P, _I64, _INT, _I32, _P, _P, _SZ, _P]),
    "ssc_select_index_i64": (_INT, [_P, _P, _I64, _INT, _I32, _P, _P, _SZ, _P]),
    "ssc_status_str": (ctypes.c_char_p, [_INT]),
    "ssc_last_hip_error": (_INT, []),
}


class SSCError(RuntimeError):
    def __init__(self, call: str, status: int, detail: str):
        super().__init__(f"{call} failed: {STATUS.get(status, status)} ({detail})")
        self.status = status


_lib = None


def load_library(path: str) -> ctypes.CDLL:
    """Load a build of the C ABI at `path` with every declared signature set."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m scan_stream_compaction_amd.build` (there is no fallback)")
    L = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib() -> ctypes.CDLL:
    """Load libssc.so (built in-tree by ``python -m scan_stream_compaction_amd.build``),
    or the build of the same sources that the environment variable
    SSC_LIBRARY names (the race checks run the whole suite through
    libssc_perturb.so that way)."""
    global _lib
    if _lib is None:
        _lib = load_library(os.environ.get("SSC_LIBRARY") or LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Route every call of this module through another build of the same
    sources (the race tests use libssc_perturb.so) while the block runs."""
    global _lib
    saved = lib()
    _lib = load_library(path)
    try:
        yield _lib
    finally:
        _lib = saved


def _check(call: str, rc: int) -> None:
    if rc != 0:
        L = lib()
        detail = L.ssc_status_str(rc).decode()
        if rc == 5:
            detail += f", hipError {L.ssc_last_hip_error()}"
        raise SSCError(call, rc, detail)


_recording = None  # list of library calls being recorded by prepared(), or None


def _call(name: str, fn, *args) -> None:
    """Make one library call (and record it while prepared() is recording).
    Tensor arguments are passed as their device pointers; a recording keeps
    the tensors themselves, so every buffer a recorded call touches (scratch
    an op allocated for itself included) lives as long as the recording."""
    raw = tuple(a.data_ptr() if isinstance(a, torch.Tensor) else a for a in args)
    if _recording is not None:
        _recording.append((name, fn, raw, args))
    _check(name, fn(*raw))


def prepared(op, *args, **kwargs):
    """Run op(*args, **kwargs) once and return a callable that repeats the
    same library calls (same buffers, same stream) with their arguments
    already marshalled: for timing loops, where the per-call Python work of
    the ops would otherwise leave the GPU waiting between launches. The
    callable returns what op returned; tensors it allocated stay alive with it.
    """
    global _recording
    calls = []
    _recording = calls
    try:
        result = op(*args, **kwargs)
    finally:
        _recording = None

    def run():
        for name, fn, raw, _ in calls:
            _check(name, fn(*raw))
        return result
    return run


def _typed(x: torch.Tensor, op: str) -> str:
    """The library entry point of `op` for x's element type."""
    if x.dtype == torch.int32:
        return f"ssc_{op}_i32"
    if x.dtype == torch.float32:
        return f"ssc_{op}_f32"
    raise TypeError(f"{op} takes int32 or float32")


def _pred(p) -> int:
    return PRED[p] if isinstance(p, str) else int(p)


def _dev(t: torch.Tensor) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("arguments must be torch tensors")
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU (no CPU path)")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")


def _need(t, name: str, like: torch.Tensor, dtypes, numel: int) -> torch.Tensor:
    """Checks a caller-supplied tensor before its device pointer reaches the
    library (which can check only alignment and overlap): a contiguous GPU
    tensor on the same device as `like`, of one of `dtypes` (None: any), with
    at least `numel` elements. Raises TypeError or ValueError otherwise."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (no CPU path)")
    if t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, the input on {like.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} must be of dtype {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements; this call needs {numel}")
    return t


def _scratch(scratch, like: torch.Tensor, nbytes: int) -> torch.Tensor:
    return _need(scratch, "scratch", like, (torch.uint8,), nbytes)


def _count(count, like: torch.Tensor) -> torch.Tensor:
    if count is None:
        return torch.empty(1, dtype=torch.int32, device=like.device)
    return _need(count, "count", like, (torch.int32,), 1)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def tile_elems() -> int:
    return int(lib().ssc_tile_elems())


def scratch_bytes(n: int) -> int:
    return int(lib().ssc_scratch_bytes(n))


def radix_sort_scratch_bytes(n: int) -> int:
    return int(lib().ssc_radix_sort_scratch_bytes(n))


def new_scratch(n: int, device, radix: bool = False) -> torch.Tensor:
    """A zero-filled scratch buffer for calls on up to n elements. The library
    keeps it ready between calls; reuse it for calls on one stream."""
    nbytes = radix_sort_scratch_bytes(n) if radix else scratch_bytes(n)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def exclusive_scan(x: torch.Tensor, out: torch.Tensor | None = None,
                   total: torch.Tensor | None = None, scratch: torch.Tensor | None = None):
    """(out, total): exclusive scan of int32 (wrapping) or float32 values."""
    return _scan(x, out, total, scratch, "exclusive")


def inclusive_scan(x: torch.Tensor, out: torch.Tensor | None = None,
                   total: torch.Tensor | None = None, scratch: torch.Tensor | None = None):
    """(out, total): inclusive scan of int32 (wrapping) or float32 values."""
    return _scan(x, out, total, scratch, "inclusive")


def _scan(x, out, total, scratch, form):
    _dev(x)
    names = {torch.int32: f"ssc_{form}_scan_i32", torch.float32: f"ssc_{form}_scan_f32"}
    if x.dtype not in names:
        raise TypeError(f"{form}_scan takes int32 or float32")
    n = x.numel()
    out = torch.empty_like(x) if out is None else _need(out, "out", x, (x.dtype,), n)
    total = (torch.empty(1, dtype=x.dtype, device=x.device) if total is None
             else _need(total, "total", x, (x.dtype,), 1))
    scratch = new_scratch(n, x.device) if scratch is None else _scratch(scratch, x, scratch_bytes(n))
    fn = (names[x.dtype], getattr(lib(), names[x.dtype]))
    _call(fn[0], fn[1], x, out, n, total, scratch,
          scratch.numel(), _stream(x))
    return out, total


def compact(x: torch.Tensor, pred="nonzero", pa: int = 0, pb: int = 0, *,
            out: torch.Tensor | None = None, count: torch.Tensor | None = None,
            ranks=False, scratch: torch.Tensor | None = None):
    """(out, count[, ranks]): order-preserving compaction of int32 values
    (predicates 0..5, int arguments pa, pb), float32 values (predicates
    "f32_*", float thresholds pa, pb) or int64 values (nonzero, odd, even,
    bit_set, bit_clear; the bit 0..63 in pa).

    out[:count] holds the survivors; entries past count are not written.
    ranks=True (or a tensor) also returns the exclusive scan of the flags
    (32-bit elements only).
    """
    _dev(x)
    n = x.numel()
    if x.dtype == torch.int64:
        if ranks is not False:
            raise ValueError("ranks are for 32-bit elements")
        return _i64_op("ssc_compact_i64", x, pred, pa,
                       torch.empty_like(x) if out is None else _need(out, "out", x, (torch.int64,), n),
                       count, scratch)
    fn = _typed(x, "compact")
    out = torch.empty_like(x) if out is None else _need(out, "out", x, (x.dtype,), n)
    count = _count(count, x)
    rk = None
    if ranks is True:
        rk = torch.empty(n, dtype=torch.int32, device=x.device)
    elif isinstance(ranks, torch.Tensor):
        rk = _need(ranks, "ranks", x, (torch.int32,), n)
    elif ranks is not False and ranks is not None:
        raise TypeError("ranks is True, False or an int32 tensor")
    scratch = new_scratch(n, x.device) if scratch is None else _scratch(scratch, x, scratch_bytes(n))
    _call(fn, getattr(lib(), fn),
          x, out, n, _pred(pred), pa, pb, count, rk,
          scratch, scratch.numel(), _stream(x))
    return (out, count, rk) if rk is not None else (out, count)


def compact_noalloc(x: torch.Tensor, pred="nonzero", pa: int = 0, pb: int = 0, *,
                    out: torch.Tensor, count: torch.Tensor, ranks: torch.Tensor | None = None):
    """(out, count[, ranks]) as compact() for int32, through the entry point
    that allocates nothing (its scratch is a library-owned array per GPU):
    the caller passes every output. Calls that may overlap on one GPU race."""
    _dev(x)
    if x.dtype != torch.int32:
        raise TypeError("compact_noalloc takes int32")
    n = x.numel()
    _need(out, "out", x, (torch.int32,), n)
    _need(count, "count", x, (torch.int32,), 1)
    if ranks is not None:
        _need(ranks, "ranks", x, (torch.int32,), n)
    _call("ssc_compact_i32_noalloc", lib().ssc_compact_i32_noalloc,
          x, out, n, _pred(pred), pa, pb, count, ranks, _stream(x))
    return (out, count, ranks) if ranks is not None else (out, count)


def select_index(x: torch.Tensor, pred="nonzero", pa: int = 0, pb: int = 0, *,
                 out: torch.Tensor | None = None, count: torch.Tensor | None = None,
                 scratch: torch.Tensor | None = None):
    """(idx, count): idx[:count] holds the positions of the elements for which
    the predicate holds, increasing; entries past count are not written.
    int64 values take nonzero, odd, even, bit_set and bit_clear (bit in pa)."""
    _dev(x)
    n = x.numel()
    if x.dtype == torch.int64:
        idx = (torch.empty(n, dtype=torch.int32, device=x.device) if out is None
               else _need(out, "out", x, (torch.int32,), n))
        return _i64_op("ssc_select_index_i64", x, pred, pa, idx, count, scratch)
    fn = _typed(x, "select_index")
    out = (torch.empty(n, dtype=torch.int32, device=x.device) if out is None
           else _need(out, "out", x, (torch.int32,), n))
    count = _count(count, x)
    scratch = new_scratch(n, x.device) if scratch is None else _scratch(scratch, x, scratch_bytes(n))
    _call(fn, getattr(lib(), fn),
          x, out, n, _pred(pred), pa, pb, count,
          scratch, scratch.numel(), _stream(x))
    return out, count


def partition(x: torch.Tensor, pred="even", pa: int = 0, pb: int = 0, *,
              out: torch.Tensor | None = None, count: torch.Tensor | None = None,
              scratch: torch.Tensor | None = None):
    """(out, count): stable partition, predicate-true elements first; count = K."""
    _dev(x)
    fn = _typed(x, "partition")
    n = x.numel()
    out = torch.empty_like(x) if out is None else _need(out, "out", x, (x.dtype,), n)
    count = _count(count, x)
    scratch = new_scratch(n, x.device) if scratch is None else _scratch(scratch, x, scratch_bytes(n))
    _call(fn, getattr(lib(), fn),
          x, out, n, _pred(pred), pa, pb, count,
          scratch, scratch.numel(), _stream(x))
    return out, count


def count_if(x: torch.Tensor, pred="nonzero", pa: int = 0, pb: int = 0, *,
             count: torch.Tensor | None = None,
             scratch: torch.Tensor | None = None) -> torch.Tensor:
    _dev(x)
    if x.dtype != torch.int32:
        raise TypeError("count_if takes int32")
    count = _count(count, x)
    scratch = new_scratch(0, x.device) if scratch is None else _scratch(scratch, x, scratch_bytes(0))
    _call("ssc_count_if_i32", lib().ssc_count_if_i32,
          x, x.numel(), _pred(pred), pa, pb, count, scratch,
          scratch.numel(), _stream(x))
    return count


def compact_atomic(x: torch.Tensor, pred="nonzero", pa: int = 0, pb: int = 0, *,
                   variant: int = 0, out: torch.Tensor | None = None,
                   count: torch.Tensor | None = None):
    """(out, count): unordered compaction by atomic counter (comparison only)."""
    _dev(x)
    if x.dtype != torch.int32:
        raise TypeError("compact_atomic takes int32")
    out = torch.empty_like(x) if out is None else _need(out, "out", x, (torch.int32,), x.numel())
    count = _count(count, x)
    _call("ssc_compact_atomic_i32", lib().ssc_compact_atomic_i32,
          x, out, x.numel(), _pred(pred), pa, pb, count,
          variant, _stream(x))
    return out, count


def radix_sort(x: torch.Tensor, *, out: torch.Tensor | None = None,
               tmp: torch.Tensor | None = None, scratch: torch.Tensor | None = None):
    """Ascending sort of 32-bit keys taken as unsigned (int32 storage)."""
    _dev(x)
    if x.element_size() != 4:
        raise TypeError("radix_sort takes 4-byte keys")
    n = x.numel()
    out = torch.empty_like(x) if out is None else _need(out, "out", x, None, n)
    tmp = torch.empty_like(x) if tmp is None else _need(tmp, "tmp", x, None, n)
    if out.element_size() != 4 or tmp.element_size() != 4:
        raise TypeError("out and tmp hold 4-byte keys")
    scratch = (new_scratch(n, x.device, radix=True) if scratch is None
               else _scratch(scratch, x, radix_sort_scratch_bytes(n)))
    _call("ssc_radix_sort_u32", lib().ssc_radix_sort_u32,
          x, out, tmp, n, scratch, scratch.numel(),
          _stream(x))
    return out


def radix_sort4_scratch_bytes(n: int) -> int:
    return int(lib().ssc_radix_sort4_scratch_bytes(n))


def radix_sort4(x: torch.Tensor, passes: int = 8, *, out: torch.Tensor | None = None,
                tmp: torch.Tensor | None = None, scratch: torch.Tensor | None = None):
    """Stable LSD sort of 32-bit keys taken as unsigned (int32 storage) by
    their low 4*passes bits, 4-bit digits; passes=8 sorts ascending."""
    _dev(x)
    if x.element_size() != 4:
        raise TypeError("radix_sort4 takes 4-byte keys")
    n = x.numel()
    out = torch.empty_like(x) if out is None else _need(out, "out", x, None, n)
    tmp = torch.empty_like(x) if tmp is None else _need(tmp, "tmp", x, None, n)
    if out.element_size() != 4 or tmp.element_size() != 4:
        raise TypeError("out and tmp hold 4-byte keys")
    scratch = (torch.zeros(radix_sort4_scratch_bytes(n), dtype=torch.uint8, device=x.device)
               if scratch is None else _scratch(scratch, x, radix_sort4_scratch_bytes(n)))
    _call("ssc_radix_sort4_u32", lib().ssc_radix_sort4_u32,
          x, out, tmp, n, passes, scratch,
          scratch.numel(), _stream(x))
    return out


def multipass_scratch(n: int, device) -> torch.Tensor:
    return torch.zeros(int(lib().ssc_multipass_scratch_bytes(n)), dtype=torch.uint8, device=device)


def exclusive_scan_multipass(x: torch.Tensor, out: torch.Tensor | None = None,
                             total: torch.Tensor | None = None,
                             scratch: torch.Tensor | None = None):
    """(out, total): the multi-launch int32 scan (comparison with the single pass)."""
    _dev(x)
    if x.dtype != torch.int32:
        raise TypeError("exclusive_scan_multipass takes int32")
    n = x.numel()
    out = torch.empty_like(x) if out is None else _need(out, "out", x, (torch.int32,), n)
    total = _count(total, x)
    scratch = (multipass_scratch(n, x.device) if scratch is None
               else _scratch(scratch, x, int(lib().ssc_multipass_scratch_bytes(n))))
    _call("ssc_exclusive_scan_multipass_i32", lib().ssc_exclusive_scan_multipass_i32,
          x, out, x.numel(), total, scratch,
          scratch.numel(), _stream(x))
    return out, total


def compact_multipass(x: torch.Tensor, pred="nonzero", pa: int = 0, pb: int = 0, *,
                      out: torch.Tensor | None = None, count: torch.Tensor | None = None,
                      ranks: torch.Tensor | None = None, scratch: torch.Tensor | None = None):
    """(out, count, ranks): the multi-launch int32 compaction (mark, scan,
    scatter), for comparison with the single pass."""
    _dev(x)
    if x.dtype != torch.int32:
        raise TypeError("compact_multipass takes int32")
    n = x.numel()
    out = torch.empty_like(x) if out is None else _need(out, "out", x, (torch.int32,), n)
    count = _count(count, x)
    ranks = torch.empty_like(x) if ranks is None else _need(ranks, "ranks", x, (torch.int32,), n)
    scratch = (multipass_scratch(n, x.device) if scratch is None
               else _scratch(scratch, x, int(lib().ssc_multipass_scratch_bytes(n))))
    _call("ssc_compact_multipass_i32", lib().ssc_compact_multipass_i32,
          x, out, n, _pred(pred), pa, pb, count, ranks,
          scratch, scratch.numel(), _stream(x))
    return out, count, ranks


def copy(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """out = x for 4-byte elements (the bandwidth reference)."""
    _dev(x)
    if x.element_size() != 4:
        raise TypeError("copy takes 4-byte elements")
    out = torch.empty_like(x) if out is None else _need(out, "out", x, (x.dtype,), x.numel())
    _call("ssc_copy_i32", lib().ssc_copy_i32, x, out, x.numel(), _stream(x))
    return out


def mark(x: torch.Tensor, pred="nonzero", pa: int = 0, pb: int = 0, *,
         out: torch.Tensor | None = None) -> torch.Tensor:
    """flags[i] = P(x[i]) as int32 0/1: the first launch of the multi-launch
    compaction (comparison only)."""
    _dev(x)
    if x.dtype != torch.int32:
        raise TypeError("mark takes int32")
    out = torch.empty_like(x) if out is None else _need(out, "out", x, (torch.int32,), x.numel())
    _call("ssc_mark_i32", lib().ssc_mark_i32, x, out, x.numel(), _pred(pred), pa, pb, _stream(x))
    return out


def scatter(x: torch.Tensor, ranks: torch.Tensor, pred="nonzero", pa: int = 0, pb: int = 0, *,
            out: torch.Tensor | None = None, count: torch.Tensor | None = None):
    """(out, count): out[ranks[i]] = x[i] where P(x[i]), given the exclusive
    scan of the flags: the last launch of the multi-launch compaction
    (comparison only)."""
    _dev(x)
    if x.dtype != torch.int32:
        raise TypeError("scatter takes int32")
    n = x.numel()
    _need(ranks, "ranks", x, (torch.int32,), n)
    out = torch.empty_like(x) if out is None else _need(out, "out", x, (torch.int32,), n)
    count = _count(count, x)
    _call("ssc_scatter_i32", lib().ssc_scatter_i32, x, ranks, out, n, _pred(pred), pa, pb, count,
          _stream(x))
    return out, count


def timed_out(scratch: torch.Tensor) -> bool:
    """True if a look-back wait of a call made with this scratch gave up after
    its bounded spin since the scratch was last zeroed (those calls' results
    are invalid; zero the scratch before reusing it). Synchronises with the
    scratch's device."""
    _dev(scratch)
    if scratch.dtype != torch.uint8:
        raise TypeError("scratch is a uint8 tensor")
    flag = torch.empty(1, dtype=torch.int32, device=scratch.device)
    _call("ssc_scratch_timed_out", lib().ssc_scratch_timed_out, scratch, scratch.numel(), flag,
          _stream(scratch))
    return bool(int(flag.item()))


def _i64_op(fn: str, x: torch.Tensor, pred, bit: int, out: torch.Tensor,
            count: torch.Tensor | None, scratch: torch.Tensor | None):
    n = x.numel()
    count = _count(count, x)
    scratch = new_scratch(n, x.device) if scratch is None else _scratch(scratch, x, scratch_bytes(n))
    _call(fn, getattr(lib(), fn), x, out, n, _pred(pred), bit,
          count, scratch, scratch.numel(), _stream(x))
    return out, count


def _flag_bytes(flags: torch.Tensor) -> torch.Tensor:
    _dev(flags)
    if flags.dtype == torch.bool:
        return flags.view(torch.uint8)
    if flags.dtype not in (torch.uint8, torch.int8):
        raise TypeError("flags are one byte per element (bool, uint8 or int8)")
    return flags


def compact_flags(x: torch.Tensor, flags: torch.Tensor, *, out: torch.Tensor | None = None,
                  count: torch.Tensor | None = None, scratch: torch.Tensor | None = None):
    """(out, count): the 32-bit elements of x (any 4-byte dtype, moved bit for
    bit) whose flag byte is nonzero, in input order -- compaction by a
    predicate the caller has already evaluated (e.g. a torch.bool mask).
    flags must start 4-byte aligned; out[count:] is not written."""
    _dev(x)
    if x.element_size() != 4:
        raise TypeError("compact_flags takes 4-byte elements")
    fb = _flag_bytes(flags)
    n = x.numel()
    if fb.numel() != n:
        raise ValueError("one flag byte per element")
    _need(fb, "flags", x, None, n)
    out = torch.empty_like(x) if out is None else _need(out, "out", x, None, n)
    if out.element_size() != 4:
        raise TypeError("out holds 4-byte elements")
    count = _count(count, x)
    scratch = new_scratch(n, x.device) if scratch is None else _scratch(scratch, x, scratch_bytes(n))
    _call("ssc_compact_flags_b32", lib().ssc_compact_flags_b32, x, fb,
          out, n, count, scratch, scratch.numel(), _stream(x))
    return out, count


def select_flags(flags: torch.Tensor, *, out: torch.Tensor | None = None,
                 count: torch.Tensor | None = None, scratch: torch.Tensor | None = None):
    """(idx, count): positions of the nonzero flag bytes, increasing (the
    one-pass form of torch.nonzero on a bool mask)."""
    fb = _flag_bytes(flags)
    n = fb.numel()
    out = (torch.empty(n, dtype=torch.int32, device=fb.device) if out is None
           else _need(out, "out", fb, (torch.int32,), n))
    count = _count(count, fb)
    scratch = new_scratch(n, fb.device) if scratch is None else _scratch(scratch, fb, scratch_bytes(n))
    _call("ssc_select_flags", lib().ssc_select_flags, fb, out, n,
          count, scratch, scratch.numel(), _stream(fb))
    return out, count


def compact_kv(keys: torch.Tensor, vals: torch.Tensor, pred="nonzero", pa=0, pb=0, *,
               keys_out: torch.Tensor | None = None, vals_out: torch.Tensor | None = None,
               count: torch.Tensor | None = None, scratch: torch.Tensor | None = None):
    """(keys_out, vals_out, count): the pairs whose key satisfies the
    predicate, in input order. int32 keys take predicates 0..5, float32 keys
    the "f32_*" ones; values are any 4-byte dtype, moved bit for bit."""
    _dev(keys)
    _dev(vals)
    if vals.element_size() != 4 or vals.numel() != keys.numel():
        raise ValueError("one 4-byte value per key")
    fn = _typed(keys, "compact_kv")
    n = keys.numel()
    _need(vals, "vals", keys, None, n)
    keys_out = (torch.empty_like(keys) if keys_out is None
                else _need(keys_out, "keys_out", keys, (keys.dtype,), n))
    vals_out = torch.empty_like(vals) if vals_out is None else _need(vals_out, "vals_out", keys, None, n)
    if vals_out.element_size() != 4:
        raise TypeError("vals_out holds 4-byte values")
    count = _count(count, keys)
    scratch = new_scratch(n, keys.device) if scratch is None else _scratch(scratch, keys, scratch_bytes(n))
    _call(fn, getattr(lib(), fn), keys, vals, keys_out,
          vals_out, n, _pred(pred), pa, pb, count, scratch,
          scratch.numel(), _stream(keys))
    return keys_out, vals_out, count
