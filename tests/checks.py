"""Result checkers used by the tests (host side, numpy).

They decide correctness from properties, not from a second implementation:
exact equality, "is a subsequence of", "holds the same multiset", and the
relative-error band for fp32 scans. Each one is shown to fail on planted
mistakes in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np


def first_mismatch(got, want) -> int:
    """Index of the first differing element, -1 if equal (lengths must match)."""
    got = np.asarray(got)
    want = np.asarray(want)
    if got.shape != want.shape:
        return min(got.size, want.size)
    bad = np.flatnonzero(got != want)
    return int(bad[0]) if bad.size else -1


def is_subsequence(sub, seq) -> bool:
    """True iff `sub` appears in `seq` in order (two pointers)."""
    sub = np.asarray(sub)
    seq = np.asarray(seq)
    j = 0
    m = sub.size
    if m == 0:
        return True
    for v in seq.tolist():
        if v == sub[j]:
            j += 1
            if j == m:
                return True
    return False


def same_multiset(a, b) -> bool:
    a = np.sort(np.asarray(a), kind="stable")
    b = np.sort(np.asarray(b), kind="stable")
    return a.shape == b.shape and bool(np.array_equal(a, b))


def count_out_of_order(got, want) -> int:
    """Positions where an unordered result differs from the ordered one (reported only)."""
    got = np.asarray(got)
    want = np.asarray(want)
    return int(np.count_nonzero(got != want))


def f32_scan_rel_errors(got, ref):
    """(max_rel, max_abs, ok) for |got - ref| <= 1e-5 |ref|, ref == 0 => got == 0."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    zero = ref == 0.0
    ok_zero = bool(np.all(got[zero] == 0.0))
    nz = ~zero
    rel = np.zeros_like(diff)
    rel[nz] = diff[nz] / np.abs(ref[nz])
    max_rel = float(rel.max()) if rel.size else 0.0
    max_abs = float(diff.max()) if diff.size else 0.0
    return max_rel, max_abs, ok_zero and max_rel <= 1e-5


F32_SCAN_REL_TOL = 1e-5
