"""Pins for the CPU oracle: each test checks the oracle against something other
than itself -- values the pages print, closed forms, invariants, brute force on
tiny inputs, or a library routine for a special case. All run on the CPU.
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np
import pytest

import oracle
from tests import checks

PRED_NAMES = {"NONZERO": oracle.PRED_NONZERO, "ODD": oracle.PRED_ODD,
              "EVEN": oracle.PRED_EVEN, "BIT_SET": oracle.PRED_BIT_SET,
              "BIT_CLEAR": oracle.PRED_BIT_CLEAR, "MOD_LT": oracle.PRED_MOD_LT}


def _read_golden(path):
    d = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            d[k.strip()] = [int(t) for t in v.split()]
    return d


# --- printed worked examples ------------------------------------------------

def _cis565_scan_array(g):
    """A 256-element array that agrees with every printed entry of the scan
    transcript: the 13-entry head, the 6-entry tail, and the three entries
    in[247..249] that the non-power-of-two tail fixes (its out[247..252]).
    The unprinted middle is filled with values in [0, 50) chosen so that the
    printed prefix sums hold; only the printed positions are checked."""
    n = g["size_pot"][0]
    x = np.zeros(n, np.int64)
    head, tail = g["input_head"], g["input_tail"]
    x[:len(head)] = head
    x[n - len(tail):] = tail
    npot_tail = g["scan_npot_tail"]  # out[247..252]
    s = n - len(tail) - 3           # 247
    x[s:s + 3] = np.diff(npot_tail[:4])   # in[247..249] = out[i+1] - out[i]
    # middle x[13:247] must sum to out[247] - (sum of head)
    need = npot_tail[0] - sum(head)
    m = s - len(head)
    base, extra = divmod(need, m)
    mid = np.full(m, base, np.int64)
    mid[:extra] += 1
    assert mid.min() >= 0 and mid.max() < 50
    x[len(head):s] = mid
    return x.astype(np.int32)


def test_cis565_scan_transcript(golden_dir):
    g = _read_golden(os.path.join(golden_dir, "cis565_scan_transcript.txt"))
    x = _cis565_scan_array(g)
    # exclusive: the head of the printed output is the exclusive scan of the head
    out, total = oracle.exclusive_scan_i32(np.array(g["input_head"], np.int32))
    assert out.tolist() == g["scan_pot_head"]
    out, total = oracle.exclusive_scan_i32(x)
    assert out[:13].tolist() == g["scan_pot_head"]
    assert out[-6:].tolist() == g["scan_pot_tail"]
    assert total == g["scan_pot_tail"][-1] + g["input_tail"][-1]   # 6518
    n_npot = g["size_npot"][0]
    out2, _ = oracle.exclusive_scan_i32(x[:n_npot])
    assert out2[:13].tolist() == g["scan_npot_head"]
    assert out2[-6:].tolist() == g["scan_npot_tail"]


def test_cis565_scan_transcript_inclusive(golden_dir):
    """The printed exclusive outputs fix the inclusive ones: inclusive[i] is the
    printed exclusive entry i + 1, and the last inclusive entry is the total."""
    g = _read_golden(os.path.join(golden_dir, "cis565_scan_transcript.txt"))
    x = _cis565_scan_array(g)
    inc = oracle.inclusive_scan_i32(x)
    assert inc[:12].tolist() == g["scan_pot_head"][1:13]
    assert inc[-7:-1].tolist() == g["scan_pot_tail"]
    assert inc[-1] == g["scan_pot_tail"][-1] + g["input_tail"][-1]   # 6518
    n_npot = g["size_npot"][0]
    inc2 = oracle.inclusive_scan_i32(x[:n_npot])
    assert inc2[:12].tolist() == g["scan_npot_head"][1:13]
    assert inc2[-7:-1].tolist() == g["scan_npot_tail"]


def test_cis565_compaction_transcript(golden_dir):
    g = _read_golden(os.path.join(golden_dir, "cis565_compaction_transcript.txt"))
    head = np.array(g["input_head"], np.int32)
    surv, m = oracle.compact_i32(head, oracle.PRED_NONZERO)
    # the head's 9 nonzero values are the first 9 printed survivors
    assert m == 9
    assert surv.tolist() == g["compact_pot_head"][:9]
    tail = np.array(g["input_tail"], np.int32)
    surv, m = oracle.compact_i32(tail, oracle.PRED_NONZERO)
    assert surv.tolist() == g["compact_pot_tail"][-m:]


def test_predicate_hand_cases(golden_dir):
    rows = 0
    with open(os.path.join(golden_dir, "predicate_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            xs, name, pa, pb, want = line.split()
            got = oracle.pred(int(xs), PRED_NAMES[name], int(pa), int(pb))
            assert got == int(want), line
            rows += 1
    assert rows >= 40


F32_PRED_NAMES = {"F32_NONZERO": oracle.PRED_F32_NONZERO, "F32_GT": oracle.PRED_F32_GT,
                  "F32_LT": oracle.PRED_F32_LT, "F32_IN": oracle.PRED_F32_IN}


def test_predicate_f32_hand_cases(golden_dir):
    rows = 0
    with open(os.path.join(golden_dir, "predicate_cases_f32.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            xs, name, a, b, want = line.split()
            got = oracle.pred_f32(float(xs), F32_PRED_NAMES[name], float(a), float(b))
            assert got == int(want), line
            rows += 1
    assert rows >= 30


def test_f32_ops_against_numpy_masks():
    """Compaction, partition and selection of fp32 values against numpy boolean
    masks (IEEE comparisons), on values that include NaN, +-0, +-inf and
    denormals."""
    from scan_stream_compaction_amd import workloads
    x = (workloads.unit_float32(11, 40_000) * 4 - 2).astype(np.float32)
    x[:10] = [np.nan, 0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 0.5, 1.0, -1.0]
    x[-3:] = [np.nan, 0.5, -0.0]
    cases = [(oracle.PRED_F32_NONZERO, 0.0, 0.0, x != 0),
             (oracle.PRED_F32_GT, 0.5, 0.0, x > np.float32(0.5)),
             (oracle.PRED_F32_LT, -0.25, 0.0, x < np.float32(-0.25)),
             (oracle.PRED_F32_IN, 0.0, 1.0, (x >= 0) & (x < 1)),
             (oracle.PRED_F32_GT, np.nan, 0.0, np.zeros(x.size, bool))]
    with np.errstate(invalid="ignore"):
        for pred, a, b, mask in cases:
            surv, m = oracle.compact_f32(x, pred, a, b)
            assert m == int(mask.sum())
            assert np.array_equal(surv, x[mask], equal_nan=True)
            assert np.array_equal(surv.view(np.uint32), x[mask].view(np.uint32))  # -0.0 kept as is
            out, k = oracle.partition_f32(x, pred, a, b)
            assert k == m
            assert np.array_equal(out.view(np.uint32),
                                  np.concatenate([x[mask], x[~mask]]).view(np.uint32))
            idx, mi = oracle.select_index_f32(x, pred, a, b)
            assert mi == m and np.array_equal(idx, np.flatnonzero(mask))


def test_predicate_arg_rules():
    assert oracle.pred_args_ok(oracle.PRED_BIT_SET, 31)
    assert not oracle.pred_args_ok(oracle.PRED_BIT_SET, 32)
    assert not oracle.pred_args_ok(oracle.PRED_BIT_CLEAR, -1)
    assert oracle.pred_args_ok(oracle.PRED_MOD_LT, 1, 0)
    assert not oracle.pred_args_ok(oracle.PRED_MOD_LT, 0, 0)
    assert not oracle.pred_args_ok(7)


# --- closed forms -------------------------------------------------------------

def test_scan_i32_closed_form_mod8():
    """in[i] = (i % 8) + 1 ("Day 31 scan.cu" input); out[i] = 36*floor(i/8) + r(r+1)/2."""
    n = 10_000_000
    x = (np.arange(n, dtype=np.int64) % 8 + 1).astype(np.int32)
    out, total = oracle.exclusive_scan_i32(x)
    i = np.arange(n, dtype=np.int64)
    r = i % 8
    want = 36 * (i // 8) + r * (r + 1) // 2
    assert checks.first_mismatch(out.astype(np.int64), want) == -1
    assert total == 45_000_000
    assert out[-1] == 44_999_992


def test_scan_f32_every_fourth_two_exact():
    """"Day 32 scan_2.cu": every fourth element 2.0f, total 12,500,000 < 2^24, so
    every prefix is an exact integer: out[i] = i + ceil(i/4)."""
    n = 10_000_000
    x = np.ones(n, np.float32)
    x[0::4] = 2.0
    out, total = oracle.exclusive_scan_f32(x)
    i = np.arange(n, dtype=np.int64)
    want = i + (i + 3) // 4
    assert np.array_equal(out, want.astype(np.float64))
    assert total == 12_500_000.0


def test_scan_f32_accumulates_in_double():
    """Against math.fsum (exactly rounded) at sample points: the fp64 running sum
    is within 1e-12 relative; an fp32 accumulator would be off by ~1e-4."""
    from scan_stream_compaction_amd import workloads
    x = workloads.unit_float32(0x1234, 200_000)
    out, total = oracle.exclusive_scan_f32(x)
    xd = x.astype(np.float64).tolist()
    for i in (1, 17, 1000, 65_537, 199_999):
        ref = math.fsum(xd[:i])
        assert abs(out[i] - ref) <= 1e-12 * ref
    ref = math.fsum(xd)
    assert abs(total - ref) <= 1e-12 * ref


def test_inclusive_scans_closed_forms():
    """(i % 8) + 1 gives inclusive[i] = 36*floor((i+1)/8) + r(r+1)/2 with
    r = (i+1) % 8; every fourth 2.0f gives inclusive[i] = (i+1) + ceil((i+1)/4),
    exactly in fp64 (all prefixes are integers below 2^24)."""
    n = 10_000_000
    x = (np.arange(n, dtype=np.int64) % 8 + 1).astype(np.int32)
    inc = oracle.inclusive_scan_i32(x)
    j = np.arange(1, n + 1, dtype=np.int64)
    r = j % 8
    assert checks.first_mismatch(inc.astype(np.int64), 36 * (j // 8) + r * (r + 1) // 2) == -1
    assert inc[-1] == 45_000_000
    xf = np.ones(n, np.float32)
    xf[0::4] = 2.0
    incf = oracle.inclusive_scan_f32(xf)
    assert np.array_equal(incf, (j + (j + 3) // 4).astype(np.float64))


def test_inclusive_scan_f32_accumulates_in_double():
    from scan_stream_compaction_amd import workloads
    x = workloads.unit_float32(0x4321, 100_000)
    inc = oracle.inclusive_scan_f32(x)
    xd = x.astype(np.float64).tolist()
    for i in (0, 5, 999, 65_536, 99_999):
        ref = math.fsum(xd[:i + 1])
        assert abs(inc[i] - ref) <= 1e-12 * ref


def test_inclusive_minus_exclusive_is_the_input():
    from scan_stream_compaction_amd import workloads
    x = workloads.full_int32(8, 40_003)
    inc = oracle.inclusive_scan_i32(x)
    exc, total = oracle.exclusive_scan_i32(x)
    assert np.array_equal((inc.astype(np.int64) - exc) % (1 << 32), x.astype(np.int64) % (1 << 32))
    assert inc[-1] == total
    inc2 = oracle.inclusive_scan_i32(np.array([2**31 - 1, 1, -5], np.int32))
    assert inc2.tolist() == [2**31 - 1, -2**31, 2**31 - 5]


def test_select_index_transcript_and_library_routine(golden_dir):
    """The positions of the CIS 565 head's nonzero values, and np.flatnonzero of
    the flags on a large input; indexing the input by them gives the compaction."""
    g = _read_golden(os.path.join(golden_dir, "cis565_compaction_transcript.txt"))
    head = np.array(g["input_head"], np.int32)
    idx, m = oracle.select_index_i32(head, oracle.PRED_NONZERO)
    assert idx.tolist() == [0, 1, 2, 5, 6, 7, 9, 10, 12] and m == 9
    assert head[idx].tolist() == g["compact_pot_head"][:9]
    from scan_stream_compaction_amd import workloads
    x = workloads.full_int32(17, 70_001)
    for pred, pa, pb in ((oracle.PRED_ODD, 0, 0), (oracle.PRED_MOD_LT, 100, 37),
                         (oracle.PRED_BIT_CLEAR, 31, 0)):
        idx, m = oracle.select_index_i32(x, pred, pa, pb)
        assert np.array_equal(idx, np.flatnonzero(oracle.flags(x, pred, pa, pb)))
        surv, m2 = oracle.compact_i32(x, pred, pa, pb)
        assert m == m2 and np.array_equal(x[idx], surv)
    e, m = oracle.select_index_i32(np.zeros(0, np.int32), oracle.PRED_ODD)
    assert m == 0 and e.size == 0


def test_scan_i32_wraps_modulo_2_32():
    """Two's-complement wrap: 2^31 - 1 + 1 is -2^31."""
    x = np.array([2**31 - 1, 1, 1, -5], np.int32)
    out, total = oracle.exclusive_scan_i32(x)
    assert out.tolist() == [0, 2**31 - 1, -2**31, -2**31 + 1]
    assert total == 2**31 - 4


def test_empty_inputs():
    e = np.zeros(0, np.int32)
    out, total = oracle.exclusive_scan_i32(e)
    assert out.size == 0 and total == 0
    o, t = oracle.exclusive_scan_f32(np.zeros(0, np.float32))
    assert o.size == 0 and t == 0.0
    s, m = oracle.compact_i32(e, oracle.PRED_ODD)
    assert m == 0 and s.size == 0
    p, k = oracle.partition_i32(e, oracle.PRED_ODD)
    assert k == 0 and p.size == 0
    assert oracle.radix_sort_u32(np.zeros(0, np.uint32)).size == 0


# --- invariants -------------------------------------------------------------------

@pytest.mark.parametrize("pred,pa,pb,k", [
    (oracle.PRED_NONZERO, 0, 0, 4), (oracle.PRED_ODD, 0, 0, 1 << 31),
    (oracle.PRED_EVEN, 0, 0, 10), (oracle.PRED_BIT_SET, 7, 0, 1 << 31),
    (oracle.PRED_BIT_CLEAR, 30, 0, 1 << 31), (oracle.PRED_MOD_LT, 100, 50, 1 << 31)])
def test_count_is_top_of_scan(pred, pa, pb, k):
    """"Day 33 compaction.cu": the survivor count is the last prefix plus the last flag."""
    from scan_stream_compaction_amd import workloads
    x = (workloads.hi32(99 + pred, 50_001).astype(np.int64) % k).astype(np.int32) \
        if k < (1 << 31) else workloads.full_int32(99 + pred, 50_001)
    f = oracle.flags(x, pred, pa, pb)
    ranks, top = oracle.exclusive_scan_i32(f)
    surv, m, ranks2 = oracle.compact_i32(x, pred, pa, pb, want_ranks=True)
    assert np.array_equal(ranks, ranks2)
    assert m == top == ranks[-1] + f[-1] == oracle.count(x, pred, pa, pb)
    # survivors: a subsequence of the input, all P-true, of length count
    assert checks.is_subsequence(surv, x)
    assert all(oracle.pred(int(v), pred, pa, pb) == 1 for v in surv[:2000])
    assert np.all(oracle.flags(surv, pred, pa, pb) == 1)
    # ranks are the output slots: out[rank[i]] == x[i] for every survivor
    keep = f == 1
    assert np.array_equal(surv[ranks[keep]], x[keep])


@pytest.mark.parametrize("T", [64, 256, 4096, 4097])
def test_tile_sum_identity(T):
    """Per-tile scans plus the exclusive scan of tile aggregates give the
    global scan ("Day 33 compaction.cu", scanTilesExclusive/addTileCarry;
    "CUDA Handbook ch. 13": earlier tiles' keep counts give the tile base)."""
    from scan_stream_compaction_amd import workloads
    x = workloads.uniform_below(7, 3 * 4096 + 611, 4)
    f = oracle.flags(x, oracle.PRED_NONZERO)
    ranks, total = oracle.exclusive_scan_i32(f)
    starts = np.arange(0, x.size, T)
    agg = np.add.reduceat(f.astype(np.int64), starts)
    carries, _ = oracle.exclusive_scan_i32(agg.astype(np.int32))
    assert np.array_equal(ranks[starts], carries)
    for t, s in enumerate(starts):
        local, _ = oracle.exclusive_scan_i32(f[s:s + T])
        assert np.array_equal(ranks[s:s + T], local + carries[t])
    assert total == int(agg.sum())


def test_partition_properties_and_i_minus_rank():
    """Stable partition: halves sum to N, each half keeps input order, and the
    "Day 33 compaction.cu" addressing (kept -> rank[i], rejected -> K + i - rank[i])
    reproduces the two-pass result."""
    from scan_stream_compaction_amd import workloads
    x = workloads.uniform_below(11, 40_003, 10)
    for pred, pa, pb in [(oracle.PRED_EVEN, 0, 0), (oracle.PRED_NONZERO, 0, 0),
                         (oracle.PRED_MOD_LT, 7, 3), (oracle.PRED_BIT_SET, 1, 0)]:
        out, k = oracle.partition_i32(x, pred, pa, pb)
        f = oracle.flags(x, pred, pa, pb)
        assert k == int(f.sum())
        assert out.size == x.size
        assert np.all(oracle.flags(out[:k], pred, pa, pb) == 1)
        assert np.all(oracle.flags(out[k:], pred, pa, pb) == 0)
        assert checks.is_subsequence(out[:k], x) and checks.is_subsequence(out[k:], x)
        assert checks.same_multiset(out, x)
        rank, _ = oracle.exclusive_scan_i32(f)
        i = np.arange(x.size)
        dest = np.where(f == 1, rank, k + i - rank)
        alt = np.empty_like(x)
        alt[dest] = x
        assert np.array_equal(alt, out)
        # i - rank[i] is the number of rejected elements before i
        rej_before = np.concatenate([[0], np.cumsum(1 - f)[:-1]])
        assert np.array_equal(i - rank, rej_before)


def test_keep_all_and_keep_none():
    from scan_stream_compaction_amd import workloads
    x = workloads.uniform_below(5, 10_007, 9) + 1  # 1..9, no zeros
    surv, m = oracle.compact_i32(x, oracle.PRED_NONZERO)
    assert m == x.size and np.array_equal(surv, x)       # keep-all is a copy
    surv, m = oracle.compact_i32(x * 0, oracle.PRED_NONZERO)
    assert m == 0
    out, k = oracle.partition_i32(x, oracle.PRED_NONZERO)
    assert k == x.size and np.array_equal(out, x)
    out, k = oracle.partition_i32(x, oracle.PRED_MOD_LT, 100, 0)
    assert k == 0 and np.array_equal(out, x)


# --- brute force ----------------------------------------------------------------

def _kth_survivor(xs, keep, k):
    """Second definition: linear search for the k-th kept element."""
    seen = 0
    for v, f in zip(xs, keep):
        if f:
            if seen == k:
                return v
            seen += 1
    raise IndexError


def test_brute_force_all_flag_vectors():
    """Every 0/1 mask of length n <= 10: compacting positions 1..n by NONZERO."""
    for n in range(0, 11):
        for mask in range(1 << n):
            keep = [(mask >> i) & 1 for i in range(n)]
            x = np.array([(i + 1) * keep[i] for i in range(n)], np.int32)
            surv, m = oracle.compact_i32(x, oracle.PRED_NONZERO, want_ranks=False)
            assert m == sum(keep)
            for k in range(m):
                assert surv[k] == _kth_survivor(range(1, n + 1), keep, k)
            if n:
                ranks, _ = oracle.exclusive_scan_i32(np.array(keep, np.int32))
                assert ranks.tolist() == [sum(keep[:i]) for i in range(n)]


def test_brute_force_small_value_inputs():
    """All 4^n arrays with values in [0, 4), n <= 5, every predicate kind."""
    cases = [(oracle.PRED_NONZERO, 0, 0, lambda v: v != 0),
             (oracle.PRED_ODD, 0, 0, lambda v: v in (1, 3)),
             (oracle.PRED_EVEN, 0, 0, lambda v: v in (0, 2)),
             (oracle.PRED_BIT_SET, 1, 0, lambda v: v in (2, 3)),
             (oracle.PRED_BIT_CLEAR, 1, 0, lambda v: v in (0, 1)),
             (oracle.PRED_MOD_LT, 3, 1, lambda v: v in (0, 3))]
    for n in range(1, 6):
        for tup in itertools.product(range(4), repeat=n):
            x = np.array(tup, np.int32)
            for pred, pa, pb, truth in cases:
                surv, m = oracle.compact_i32(x, pred, pa, pb)
                want = [v for v in tup if truth(v)]
                assert surv.tolist() == want
                out, k = oracle.partition_i32(x, pred, pa, pb)
                assert out.tolist() == want + [v for v in tup if not truth(v)]
                assert k == len(want)


# --- radix ------------------------------------------------------------------------

def test_radix_matches_sort_and_stable_prefix_sorts():
    """After pass b the keys are stably sorted by their low b bits; after 32
    passes they are ascending (checked against numpy's sort), and pass 1 equals
    the EVEN partition."""
    from scan_stream_compaction_amd import workloads
    x = workloads.full_uint32(42, 30_011)
    assert np.array_equal(oracle.radix_sort_u32(x), np.sort(x))
    for b in (1, 3, 8, 17, 31):
        got = oracle.radix_sort_u32(x, passes=b)
        order = np.argsort(x & np.uint32((1 << b) - 1), kind="stable")
        assert np.array_equal(got, x[order])
    p, _ = oracle.partition_i32(x.view(np.int32), oracle.PRED_EVEN)
    assert np.array_equal(oracle.radix_sort_u32(x, passes=1), p.view(np.uint32))
    small = np.array([13, 37, 15, 2, 33, 20, 18, 9, 34, 39, 33, 40, 20], np.uint32)
    assert oracle.radix_sort_u32(small).tolist() == sorted(small.tolist())


# --- a caller's predicate as flag bytes, key-value pairs, 64-bit elements -------

def test_flag_compaction_against_numpy_and_brute_force():
    """Compaction by flag bytes ("Day 33 compaction.cu": everything after the
    predicate reads an array of ones and zeros): against numpy boolean
    indexing with any nonzero byte as true, against a k-th-survivor linear
    search for every flag vector of length <= 10, and selection against
    numpy's flatnonzero."""
    from scan_stream_compaction_amd import workloads
    rng = np.random.default_rng(5)
    x = workloads.full_int32(7, 20_011)
    f = rng.integers(0, 4, x.size).astype(np.uint8) * np.uint8(85)  # 0, 85, 170, 255
    f[:6] = [0, 1, 2, 128, 255, 0]
    surv, m = oracle.compact_flags(x, f)
    assert m == int((f != 0).sum())
    assert np.array_equal(surv, x[f != 0])
    xf = x.view(np.float32)
    survf, mf = oracle.compact_flags(xf, f)
    assert mf == m and np.array_equal(survf.view(np.uint32), xf[f != 0].view(np.uint32))
    idx, mi = oracle.select_flags(f)
    assert mi == m and np.array_equal(idx, np.flatnonzero(f))
    assert np.array_equal(oracle.compact_flags(np.arange(x.size, dtype=np.int32), f)[0], idx)
    for n in range(0, 11):
        xs = list(range(100, 100 + n))
        for mask in range(1 << n):
            keep = [(mask >> i) & 1 for i in range(n)]
            fb = np.array([k * (1 + 7 * i) for i, k in enumerate(keep)], np.uint8)
            got, mm = oracle.compact_flags(np.array(xs, np.int32), fb)
            assert mm == sum(keep)
            for k in range(mm):
                assert got[k] == _kth_survivor(xs, keep, k)
            assert oracle.select_flags(fb)[0].tolist() == [i for i in range(n) if keep[i]]
    assert oracle.compact_flags(np.zeros(0, np.int32), np.zeros(0, np.uint8))[1] == 0


def test_key_value_pairs_stay_together():
    """Key-value compaction: the keys compacted are the keys numpy's mask keeps,
    and every value is the one that sat beside its key (values are a
    one-to-one function of the position, so a value out of place shows)."""
    from scan_stream_compaction_amd import workloads
    keys = workloads.full_int32(9, 30_001)
    vals = (np.arange(keys.size, dtype=np.uint32) * np.uint32(2654435761)).view(np.float32)
    cases = [(oracle.PRED_ODD, 0, 0, (keys & 1) == 1),
             (oracle.PRED_BIT_CLEAR, 30, 0, ((keys.view(np.uint32) >> 30) & 1) == 0),
             (oracle.PRED_MOD_LT, 100, 37, np.mod(keys.astype(np.int64), 100) < 37)]
    for pred, a, b, mask in cases:
        ok, ov, m = oracle.compact_kv(keys, vals, pred, a, b)
        assert m == int(mask.sum())
        assert np.array_equal(ok, keys[mask])
        assert np.array_equal(ov.view(np.uint32), vals[mask].view(np.uint32))
    fk = (workloads.unit_float32(4, 10_000) * 2 - 1).astype(np.float32)
    fk[:4] = [np.nan, -0.0, 0.0, 0.5]
    iv = np.arange(fk.size, dtype=np.int32)
    with np.errstate(invalid="ignore"):
        for pred, a, b, mask in [(oracle.PRED_F32_GT, 0.25, 0.0, fk > np.float32(0.25)),
                                 (oracle.PRED_F32_NONZERO, 0.0, 0.0, fk != 0)]:
            ok, ov, m = oracle.compact_kv(fk, iv, pred, a, b)
            assert m == int(mask.sum())
            assert np.array_equal(ok.view(np.uint32), fk[mask].view(np.uint32))
            assert np.array_equal(ov, np.flatnonzero(mask))


I64_PRED_NAMES = {"NONZERO": oracle.PRED_NONZERO, "ODD": oracle.PRED_ODD,
                  "EVEN": oracle.PRED_EVEN, "BIT_SET": oracle.PRED_BIT_SET,
                  "BIT_CLEAR": oracle.PRED_BIT_CLEAR}


def test_predicate_i64_hand_cases(golden_dir):
    rows = 0
    with open(os.path.join(golden_dir, "predicate_cases_i64.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            xs, name, b, want = line.split()
            got = oracle.pred_i64(int(xs), I64_PRED_NAMES[name], int(b))
            assert got == int(want), line
            rows += 1
    assert rows >= 35
    assert oracle.pred_args_ok_i64(oracle.PRED_BIT_SET, 63)
    assert not oracle.pred_args_ok_i64(oracle.PRED_BIT_SET, 64)
    assert not oracle.pred_args_ok_i64(oracle.PRED_BIT_CLEAR, -1)
    assert not oracle.pred_args_ok_i64(oracle.PRED_MOD_LT, 100)


def test_i64_ops_against_numpy_bits():
    """64-bit compaction and selection against numpy's bit arithmetic on the
    unsigned view, for bits on both sides of the 32-bit boundary; values in
    int32 range with bits below 31 agree with the (pinned) int32 oracle."""
    rng = np.random.default_rng(8)
    x = rng.integers(-2**63, 2**63 - 1, 25_000, dtype=np.int64, endpoint=True)
    x[:5] = [-2**63, -1, 0, 2**63 - 1, 2**32]
    u = x.view(np.uint64)
    cases = [(oracle.PRED_NONZERO, 0, x != 0), (oracle.PRED_ODD, 0, (u & 1) == 1),
             (oracle.PRED_EVEN, 0, (u & 1) == 0)]
    for b in (0, 5, 31, 32, 33, 47, 62, 63):
        cases.append((oracle.PRED_BIT_SET, b, ((u >> np.uint64(b)) & 1) == 1))
        cases.append((oracle.PRED_BIT_CLEAR, b, ((u >> np.uint64(b)) & 1) == 0))
    for pred, b, mask in cases:
        surv, m = oracle.compact_i64(x, pred, b)
        assert m == int(mask.sum()) and np.array_equal(surv, x[mask])
        idx, mi = oracle.select_index_i64(x, pred, b)
        assert mi == m and np.array_equal(idx, np.flatnonzero(mask))
    small = rng.integers(-2**31, 2**31, 5_000, dtype=np.int64)
    for pred, b in [(oracle.PRED_ODD, 0), (oracle.PRED_BIT_SET, 7), (oracle.PRED_BIT_CLEAR, 30)]:
        assert np.array_equal(oracle.compact_i64(small, pred, b)[0],
                              oracle.compact_i32(small.astype(np.int32), pred, b)[0])


# --- the checkers themselves fail on planted mistakes ---------------------------

def test_checkers_catch_planted_mistakes():
    from scan_stream_compaction_amd import workloads
    x = workloads.uniform_below(3, 5_000, 4)
    want, m = oracle.compact_i32(x, oracle.PRED_NONZERO)
    assert checks.first_mismatch(want, want) == -1
    bad = want.copy(); bad[100] ^= 1
    assert checks.first_mismatch(bad, want) == 100
    swap = want.copy(); swap[[10, 11]] = swap[[11, 10]]
    if swap[10] != swap[11]:
        assert checks.first_mismatch(swap, want) == 10
    i = int(np.flatnonzero(want[1:] != want[:-1])[0])
    swap = want.copy(); swap[[i, i + 1]] = swap[[i + 1, i]]
    assert not checks.is_subsequence(swap, x) or checks.first_mismatch(swap, want) != -1
    assert checks.same_multiset(swap, want)
    assert not checks.same_multiset(want[:-1], want)
    assert not checks.same_multiset(bad, want)
    assert checks.is_subsequence(want, x)
    assert not checks.is_subsequence(np.append(want, 7), x)
    # the fp32 band
    ref = np.array([0.0, 1.0, 10.0])
    assert checks.f32_scan_rel_errors(ref, ref)[2]
    assert not checks.f32_scan_rel_errors(ref * (1 + 2e-5), ref)[2]
    assert not checks.f32_scan_rel_errors(np.array([1e-30, 1.0, 10.0]), ref)[2]
