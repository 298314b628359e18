"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer results must match bit for bit; fp32 scans must be within 1e-5
relative of the fp64 oracle (bit-exact where every prefix is an exact
integer below 2^24). The unordered atomic compaction is checked as a
multiset. Inputs come from the seeded generators in
scan_stream_compaction_amd.workloads, at the five workloads' full sizes and
at edge sizes around the 30720-element tile, the compaction kernel's
2048-element wavefront chunks, and the scan kernel's 15360-element rounds
and 1024-element chunks; also at more tiles than the persistent compaction
kernel has workgroups (one per compute unit).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import scan_stream_compaction_amd as ssc
from scan_stream_compaction_amd import workloads as wl
from tests import checks

pytestmark = pytest.mark.gpu

T = 30720   # elements per tile (one claim)
S = 15360   # elements per round (15 data wavefronts x 1024)
C = 1024    # elements per wavefront chunk (scan kernel)
C2 = 2048   # elements per wavefront chunk (compaction kernel)
SENTINEL = -123456789
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_compact(x: np.ndarray, pred, pa=0, pb=0, ranks=True, xd=None):
    """Run the GPU compaction and compare out/count/ranks with the oracle."""
    p = ssc.PRED[pred] if isinstance(pred, str) else pred
    want, m, want_ranks = oracle.compact_i32(x, p, pa, pb, want_ranks=True)
    xd = dev(x) if xd is None else xd
    out = torch.full_like(xd, SENTINEL)
    res = ssc.compact(xd, p, pa, pb, out=out, ranks=ranks)
    got_m = int(host(res[1])[0])
    assert got_m == m, (pred, pa, pb, got_m, m)
    o = host(out)
    assert checks.first_mismatch(o[:m], want) == -1
    assert np.all(o[m:] == SENTINEL), "compaction wrote past count"
    if ranks:
        assert checks.first_mismatch(host(res[2]), want_ranks) == -1
    return m


def check_partition(x: np.ndarray, pred, pa=0, pb=0, xd=None):
    p = ssc.PRED[pred] if isinstance(pred, str) else pred
    want, k = oracle.partition_i32(x, p, pa, pb)
    xd = dev(x) if xd is None else xd
    out, cnt = ssc.partition(xd, p, pa, pb)
    assert int(host(cnt)[0]) == k
    assert checks.first_mismatch(host(out), want) == -1
    return k


def check_scan_i32(x: np.ndarray):
    want, total = oracle.exclusive_scan_i32(x)
    out, tot = ssc.exclusive_scan(dev(x))
    assert checks.first_mismatch(host(out), want) == -1
    assert int(host(tot)[0]) == total


def check_scan_f32(x: np.ndarray, exact=False):
    ref, ref_total = oracle.exclusive_scan_f32(x)
    out, tot = ssc.exclusive_scan(dev(x))
    got = host(out)
    if exact:
        assert checks.first_mismatch(got.astype(np.float64), ref) == -1
        assert float(host(tot)[0]) == ref_total
        return 0.0
    max_rel, max_abs, ok = checks.f32_scan_rel_errors(got, ref)
    say(f"  f32 scan n={x.size}: max rel err {max_rel:.3e}, max abs err {max_abs:.3e}")
    assert ok, (max_rel, max_abs)
    t = float(host(tot)[0])
    assert abs(t - ref_total) <= checks.F32_SCAN_REL_TOL * abs(ref_total)
    return max_rel


def check_inclusive_i32(x: np.ndarray, xd=None, out=None):
    want = oracle.inclusive_scan_i32(x)
    xd = dev(x) if xd is None else xd
    got, tot = ssc.inclusive_scan(xd, out=out)
    assert checks.first_mismatch(host(got), want) == -1
    assert int(host(tot)[0]) == (int(want[-1]) if x.size else 0)


def check_inclusive_f32(x: np.ndarray, exact=False):
    ref = oracle.inclusive_scan_f32(x)
    out, tot = ssc.inclusive_scan(dev(x))
    got = host(out)
    if exact:
        assert checks.first_mismatch(got.astype(np.float64), ref) == -1
        return 0.0
    max_rel, max_abs, ok = checks.f32_scan_rel_errors(got, ref)
    say(f"  inclusive f32 scan n={x.size}: max rel err {max_rel:.3e}, max abs err {max_abs:.3e}")
    assert ok, (max_rel, max_abs)
    if x.size:
        assert abs(float(host(tot)[0]) - ref[-1]) <= checks.F32_SCAN_REL_TOL * abs(ref[-1])
    return max_rel


def check_select_index(x: np.ndarray, pred, pa=0, pb=0, xd=None):
    """Indices of the survivors against the oracle; idx past count untouched."""
    p = ssc.PRED[pred] if isinstance(pred, str) else pred
    want, m = oracle.select_index_i32(x, p, pa, pb)
    xd = dev(x) if xd is None else xd
    idx = torch.full_like(xd, SENTINEL)
    _, cnt = ssc.select_index(xd, p, pa, pb, out=idx)
    assert int(host(cnt)[0]) == m, (pred, pa, pb)
    o = host(idx)
    assert checks.first_mismatch(o[:m], want) == -1
    assert np.all(o[m:] == SENTINEL), "selection wrote past count"
    return m


# ------------------------------------------------------------ device check ---

def test_device_is_gfx950_wave64():
    assert torch.cuda.is_available(), "no GPU visible"
    props = torch.cuda.get_device_properties(0)
    say("device:", props.name, getattr(props, "gcnArchName", "?"))
    assert "gfx950" in getattr(props, "gcnArchName", "")
    assert ssc.tile_elems() == T


# ------------------------------------------------------- the five workloads ---

def test_small_compaction_with_ranks():
    """65,533 int32 in [0, 4), zeros removed; out, count and the exclusive scan of flags."""
    x = wl.small_compact_input()
    m = check_compact(x, "nonzero")
    say(f"  kept {m} of {x.size}")
    assert 0.70 * x.size < m < 0.80 * x.size


def test_zero_removal_then_partition():
    """8,387,997 int32 in [0, 10): zero removal, even/odd partition of the same
    input, and the chained form partition(compact(x))."""
    x = wl.zero_removal_input()
    xd = dev(x)
    m = check_compact(x, "nonzero", xd=xd)
    k = check_partition(x, "even", xd=xd)
    say(f"  nonzero kept {m}, even first half {k} of {x.size}")
    survivors, _ = oracle.compact_i32(x, oracle.PRED_NONZERO)
    out, cnt = ssc.compact(xd, "nonzero")
    chained, kc = ssc.partition(out[: int(host(cnt)[0])].contiguous(), "even")
    want, kw = oracle.partition_i32(survivors, oracle.PRED_EVEN)
    assert int(host(kc)[0]) == kw
    assert checks.first_mismatch(host(chained), want) == -1


def test_scan_i32_mod8():
    """10^7 int32 (i % 8) + 1: bit-exact, and against the closed form."""
    x = wl.mod8_plus1(wl.N_SCAN)
    out, tot = ssc.exclusive_scan(dev(x))
    got = host(out).astype(np.int64)
    i = np.arange(x.size, dtype=np.int64)
    r = i % 8
    assert checks.first_mismatch(got, 36 * (i // 8) + r * (r + 1) // 2) == -1
    assert int(host(tot)[0]) == 45_000_000
    check_scan_i32(x)


def test_scan_f32_uniform():
    """10^7 fp32 uniform in [0, 1): within 1e-5 relative of the fp64 oracle."""
    check_scan_f32(wl.scan_f32_input())


def test_scan_f32_every_fourth_two_exact():
    """Every prefix is an integer below 2^24, so any order of additions is exact."""
    check_scan_f32(wl.every_fourth_two(wl.N_SCAN), exact=True)


def test_inclusive_scans_full_size():
    """10^7 int32 (i % 8) + 1 bit-exact (closed form 36*floor((i+1)/8) + r(r+1)/2,
    r = (i+1) % 8); fp32 uniform within 1e-5; every fourth 2.0f bit-exact."""
    x = wl.mod8_plus1(wl.N_SCAN)
    out, tot = ssc.inclusive_scan(dev(x))
    j = np.arange(1, x.size + 1, dtype=np.int64)
    r = j % 8
    assert checks.first_mismatch(host(out).astype(np.int64), 36 * (j // 8) + r * (r + 1) // 2) == -1
    assert int(host(tot)[0]) == 45_000_000
    check_inclusive_i32(x)
    check_inclusive_f32(wl.scan_f32_input())
    check_inclusive_f32(wl.every_fourth_two(wl.N_SCAN), exact=True)


def test_scan_f32_error_does_not_grow_with_tiles():
    """2^27 fp32 uniform [0, 1) (4,370 tiles): with fp64 carries between tiles
    every output stays within 4e-7 relative of the fp64 oracle, exclusive and
    inclusive (fp32 carries measured 9.4e-7 at this size, 2.5e-7 at 10^7)."""
    x = wl.unit_float32(0x77, 1 << 27)
    xd = dev(x)
    ref, ref_total = oracle.exclusive_scan_f32(x)
    out, tot = ssc.exclusive_scan(xd)
    max_rel, _, ok = checks.f32_scan_rel_errors(host(out), ref)
    say(f"  exclusive f32 n=2^27: max rel err {max_rel:.3e}")
    assert ok and max_rel <= 4e-7, max_rel
    assert abs(float(host(tot)[0]) - ref_total) <= 4e-7 * ref_total
    del out
    ref_inc = oracle.inclusive_scan_f32(x)
    out, tot = ssc.inclusive_scan(xd)
    max_rel, _, ok = checks.f32_scan_rel_errors(host(out), ref_inc)
    say(f"  inclusive f32 n=2^27: max rel err {max_rel:.3e}")
    assert ok and max_rel <= 4e-7, max_rel


def test_inclusive_scan_wraps_and_in_place():
    x = wl.full_int32(5, 3 * T + 17)
    x[:3] = [2**31 - 1, 1, -5]
    check_inclusive_i32(x)
    xd = dev(x)
    check_inclusive_i32(x, xd=xd.clone(), out=None)
    y = xd.clone()
    ssc.inclusive_scan(y, out=y)
    assert checks.first_mismatch(host(y), oracle.inclusive_scan_i32(x)) == -1


@pytest.fixture(scope="module")
def headline():
    say("  generating 2^28 full-range int32 ...")
    x = wl.headline_input()
    xd = dev(x)
    return x, xd


def test_headline_odd_compaction_full_size(headline):
    """2^28 int32, predicate odd: the exact launch the benchmark times."""
    x, xd = headline
    m = check_compact(x, "odd", xd=xd, ranks=False)
    say(f"  odd kept {m} of {x.size} ({m / x.size:.4f})")


def test_headline_odd_selection_full_size(headline):
    """2^28 int32, predicate odd: the positions of the survivors."""
    x, xd = headline
    m = check_select_index(x, "odd", xd=xd)
    say(f"  odd selected {m} of {x.size}")


def test_maximum_size_compaction_and_selection():
    """n = 2^31 - 1, the largest n the C ABI takes (8 GiB in and out), for
    compaction, selection (by predicate and by flag bytes) and the scan: byte
    offsets past 4 GiB, tile numbers near the descriptor capacity, and a
    count near 2^30; compared element by element with the full oracle."""
    n = 2**31 - 1
    say("  generating 2^31 - 1 full-range int32 ...")
    x = wl.full_int32(0x5EED0107, n)
    want, m = oracle.compact_i32(x, oracle.PRED_ODD)
    xd = dev(x)
    out = torch.empty_like(xd)
    out[-1] = SENTINEL
    _, cnt = ssc.compact(xd, "odd", out=out)
    assert int(host(cnt)[0]) == m
    got = host(out)
    assert checks.first_mismatch(got[:m], want) == -1
    assert got[-1] == SENTINEL or m == n
    del got, want
    idx = out  # reuse the 8 GiB buffer for the positions
    _, cnt = ssc.select_index(xd, "odd", out=idx)
    assert int(host(cnt)[0]) == m
    wi, mi = oracle.select_index_i32(x, oracle.PRED_ODD)
    assert mi == m and checks.first_mismatch(host(idx)[:m], wi) == -1
    say(f"  kept {m} of {n}")
    # the same positions by flag bytes (x & 1, 2 GiB): the large-tile kernel,
    # positions up to 2^31 - 2
    fd = (xd & 1).to(torch.uint8)
    assert fd.data_ptr() % 16 == 0
    idx.fill_(SENTINEL)
    _, cnt = ssc.select_flags(fd, out=idx)
    assert int(host(cnt)[0]) == m
    assert checks.first_mismatch(host(idx)[:m], wi) == -1
    del fd, wi
    # exclusive scan (the persistent kernel, 69,906 tiles), wrapping sums
    sw, total = oracle.exclusive_scan_i32(x)
    _, tot = ssc.exclusive_scan(xd, out=out)
    assert int(host(tot)[0]) == total
    assert checks.first_mismatch(host(out), sw) == -1


@pytest.mark.parametrize("keep", wl.SWEEP_KEEP)
def test_headline_selectivity_sweep(headline, keep):
    """Keep x when mod(x, 100) < s, s in {1, 50, 99}, on the same 2^28 array."""
    x, xd = headline
    m = check_compact(x, "mod_lt", wl.SWEEP_MOD, keep, xd=xd, ranks=False)
    say(f"  mod_lt {keep}: kept {m / x.size:.4f}")
    assert abs(m / x.size - keep / 100) < 0.01


@pytest.mark.parametrize("pred,pa,pb", [("odd", 0, 0), ("mod_lt", 100, 1), ("mod_lt", 100, 99)])
def test_headline_atomic_is_same_multiset(headline, pred, pa, pb):
    x, xd = headline
    p = ssc.PRED[pred]
    want, m = oracle.compact_i32(x, p, pa, pb)
    out, cnt = ssc.compact_atomic(xd, p, pa, pb, variant=0)
    assert int(host(cnt)[0]) == m
    got_sorted = torch.sort(out[:m])[0]
    want_sorted = torch.sort(dev(want))[0]
    assert torch.equal(got_sorted, want_sorted)
    ooo = checks.count_out_of_order(host(out[:m]), want)
    say(f"  atomic {pred} {pb}: {ooo} of {m} positions out of order (reported only)")


def test_radix_sort_full_size():
    """2^24 uint32 keys, 32 chained bit-clear partitions vs numpy's sort and the oracle."""
    x = wl.radix_input()
    got = host(ssc.radix_sort(dev(x.view(np.int32)))).view(np.uint32)
    assert checks.first_mismatch(got, np.sort(x)) == -1
    assert checks.first_mismatch(got, oracle.radix_sort_u32(x)) == -1


R4 = 8192  # keys per tile of the 4-bit radix sort


def test_radix4_full_size():
    """2^24 uint32 keys, 8 passes of 4-bit digits vs numpy's sort and the oracle."""
    x = wl.radix_input()
    got = host(ssc.radix_sort4(dev(x.view(np.int32)))).view(np.uint32)
    assert checks.first_mismatch(got, np.sort(x)) == -1
    assert checks.first_mismatch(got, oracle.radix_sort_u32(x)) == -1


@pytest.mark.parametrize("n", [3 * R4 + 1234, 100_003])
def test_radix4_partial_passes_match_the_bit_split_oracle(n):
    """After p 4-bit passes the keys must equal the oracle's state after 4p
    one-bit splits: stably sorted by the low 4p bits, equal low bits kept in
    input order (stability is visible because the high bits differ)."""
    x = wl.full_uint32(0x5EED0105 + n, n)
    xd = dev(x.view(np.int32))
    for p in range(1, 9):
        got = host(ssc.radix_sort4(xd, passes=p)).view(np.uint32)
        want = oracle.radix_sort_u32(x, passes=4 * p)
        assert checks.first_mismatch(got, want) == -1, (n, p)


@pytest.mark.parametrize("n", [0, 1, 2, 63, 64, 65, 1023, 1024, 1025, R4 - 1, R4, R4 + 1,
                               2 * R4 - 1, 2 * R4 + 1, 7 * R4 + 611])
def test_radix4_edge_sizes(n):
    x = wl.full_uint32(0x5EED0205 + n, n)
    got = host(ssc.radix_sort4(dev(x.view(np.int32)))).view(np.uint32)
    assert checks.first_mismatch(got, np.sort(x)) == -1
    # few distinct digits: every lane of a wavefront shares a digit with many others
    y = wl.uniform_below(0x5EED0305 + n, n, 16).view(np.uint32) * np.uint32(0x11111111)
    got = host(ssc.radix_sort4(dev(y.view(np.int32)), passes=3)).view(np.uint32)
    assert checks.first_mismatch(got, oracle.radix_sort_u32(y, passes=12)) == -1


def test_radix4_reuses_one_scratch_across_sizes_and_passes():
    """The sort keeps state in its scratch between calls (digit counters that
    end each call at zero, the tile counter and its epoch): calls of
    different sizes and pass counts on one zero-filled scratch all match."""
    big = 100_003
    scratch = torch.zeros(ssc.radix_sort4_scratch_bytes(big), dtype=torch.uint8, device=DEV)
    for i, (n, p) in enumerate([(big, 8), (5000, 3), (big, 5), (2 * R4, 8), (1, 1), (big, 8)]):
        x = wl.full_uint32(0x5EED0505 + i, n)
        got = host(ssc.radix_sort4(dev(x.view(np.int32)), passes=p, scratch=scratch)).view(np.uint32)
        assert checks.first_mismatch(got, oracle.radix_sort_u32(x, passes=4 * p)) == -1, (n, p)


def test_radix4_unaligned_in_place_and_odd_passes():
    n = 5 * R4 + 77
    x = wl.full_uint32(0x5EED0405, n)
    # 4-byte but not 16-byte aligned arrays take the 32-bit path
    base = torch.empty(n + 1, dtype=torch.int32, device=DEV)
    base[1:] = dev(x.view(np.int32))
    out = torch.empty(n + 1, dtype=torch.int32, device=DEV)[1:]
    tmp = torch.empty(n + 1, dtype=torch.int32, device=DEV)[1:]
    got = host(ssc.radix_sort4(base[1:], passes=5, out=out, tmp=tmp)).view(np.uint32)
    assert checks.first_mismatch(got, oracle.radix_sort_u32(x, passes=20)) == -1
    assert checks.first_mismatch(host(base[1:]).view(np.uint32), x) == -1, "input modified"
    # out == in with an even number of passes
    xd = dev(x.view(np.int32))
    ssc.radix_sort4(xd, passes=8, out=xd)
    assert checks.first_mismatch(host(xd).view(np.uint32), np.sort(x)) == -1
    with pytest.raises(ssc.SSCError):
        ssc.radix_sort4(xd, passes=7, out=xd)
    with pytest.raises(ssc.SSCError):
        ssc.radix_sort4(xd, passes=0)


# -------------------------------------------------------------- edge cases ---

EDGE_N = [0, 1, 2, 3, 5, 63, 64, 65, 255, 256, 257, C - 1, C, C + 1, C2 - 1, C2, C2 + 1,
          7 * C + 3, 14 * C2 - 1, 14 * C2 + 1, S - 1, S, S + 1, T - 1, T, T + 1, 2 * T - 1, 2 * T,
          2 * T + 1, 3 * T + 2 * C2 + 1, 5 * T + 611, 64 * T + 13, 65 * T + T - 1, 700 * T + 17]


@pytest.mark.parametrize("n", EDGE_N)
def test_edge_sizes_all_ops(n):
    x = wl.uniform_below(1000 + n, n, 10)
    check_compact(x, "nonzero")
    check_compact(x, "odd")
    check_partition(x, "even")
    check_scan_i32(x)
    check_inclusive_i32(x)
    check_select_index(x, "odd")
    check_scan_f32(wl.unit_float32(2000 + n, n))
    got = ssc.count_if(dev(x), "odd")
    assert int(host(got)[0]) == oracle.count(x, oracle.PRED_ODD)
    cp = ssc.copy(dev(x))
    assert checks.first_mismatch(host(cp), x) == -1


PRED_CASES = [("nonzero", 0, 0), ("odd", 0, 0), ("even", 0, 0), ("bit_set", 0, 0),
              ("bit_set", 13, 0), ("bit_set", 31, 0), ("bit_clear", 0, 0),
              ("bit_clear", 31, 0), ("mod_lt", 100, 50), ("mod_lt", 7, 3), ("mod_lt", 1, 1),
              ("mod_lt", 2147483647, 5), ("mod_lt", 3, 0),
              # moduli from 2 to 2^31 - 2 for the residue test read off a
              # fraction: powers of two, 2^30 + 1, large primes, bounds <= 0 or >= m
              ("mod_lt", 2, 1), ("mod_lt", 16, 5), ("mod_lt", 641, 320), ("mod_lt", 65535, 100),
              ("mod_lt", 1 << 30, 7), ("mod_lt", (1 << 30) + 1, 1 << 29),
              ("mod_lt", 1000000007, 123456789), ("mod_lt", 2147483646, 1073741823),
              ("mod_lt", 3, -1), ("mod_lt", 100, 100), ("mod_lt", 5, 2147483647)]


@pytest.mark.parametrize("pred,pa,pb", PRED_CASES)
def test_every_predicate_full_range(pred, pa, pb):
    x = wl.full_int32(77, 3 * T + 611)
    x[:8] = [0, -1, 1, -2147483648, 2147483647, -3, 4, -100]
    check_compact(x, pred, pa, pb)
    check_partition(x, pred, pa, pb)
    check_select_index(x, pred, pa, pb)
    want, m = oracle.compact_i32(x, ssc.PRED[pred], pa, pb)
    out, cnt = ssc.compact_atomic(dev(x), pred, pa, pb, variant=1)
    assert int(host(cnt)[0]) == m
    assert checks.same_multiset(host(out)[:m], want)


MOD_EDGE_CASES = [(1, 1), (3, 2), (100, 1), (100, 99), ((1 << 20) + 1, 1 << 19), (1000000007, 3),
                  (2147483647, 2147483646), (2147483647, 1)]


@pytest.mark.parametrize("m,s", MOD_EDGE_CASES)
def test_mod_lt_at_residue_edges(m, s):
    """MOD_LT where the residue test is tightest: every value has residue 0,
    s - 1, s or m - 1 (the fractions nearest the threshold s/m and nearest 0
    and 1), with quotients at both ends of the int32 range and around 0,
    where the rounding error of the fraction is largest or the sign flips."""
    lo, hi = -(1 << 31), (1 << 31) - 1
    qs = set()
    for q0 in (lo // m, 0, hi // m):
        qs.update(range(q0 - 40, q0 + 41))
    rs = sorted({0, max(s - 1, 0), min(s, m - 1), m - 1})
    vals = [q * m + r for q in sorted(qs) for r in rs]
    x = np.array([v for v in vals if lo <= v <= hi], dtype=np.int64).astype(np.int32)
    x = np.concatenate([x, np.array([lo, hi, 0, -1, 1], np.int32)])
    reps = -(-(T + 97) // x.size)  # several tiles, a ragged tail
    x = np.tile(x, reps)[: T + 97 + x.size]
    check_compact(x, "mod_lt", m, s)
    check_compact(x, "mod_lt", m, s, ranks=False)
    check_select_index(x, "mod_lt", m, s)


# MOD_LT(m, s) takes one of two kernel forms by the fraction s/m it would keep
# of uniform input (dense from 3/4); each form must be right whatever the
# input keeps, and so must the run writes, whose second half of stores is
# issued only for runs longer than half a chunk.
MOD_FORM_CASES = [(m, s, keep) for m, s in [(100, 1), (100, 6), (16, 1), (100, 7), (100, 50),
                                            (100, 75), (100, 99), (4, 3), (1, 1)]
                  for keep in ("none", "all", "runs") if not (s >= m and keep == "none")]


@pytest.mark.parametrize("m,s,keep", MOD_FORM_CASES)
def test_mod_lt_forms_whatever_the_input_keeps(m, s, keep):
    n = 3 * T + 4097
    # values q*m + r have residue r (0 <= r < m) for every quotient q
    q = wl.full_int32(0x5EED0D00 + m + s, n).astype(np.int64) // max(m, 2)
    kept_r, dropped_r = 0, min(s, m - 1)  # dropped_r is kept too when s >= m
    if keep == "none":
        r = np.full(n, dropped_r)
    elif keep == "all":
        r = np.full(n, kept_r)
    else:  # alternating runs of 1 to 5000 kept and dropped values
        rng = np.random.default_rng(0x5EED0D80 + m + s)
        lens = rng.integers(1, 5001, size=n // 2 + 1)
        sel = np.repeat(np.arange(lens.size) % 2, lens)[:n]
        r = np.where(sel == 0, kept_r, dropped_r)
    x = np.clip(q * m + r, -(1 << 31), (1 << 31) - 1).astype(np.int32)
    kept = check_compact(x, "mod_lt", m, s, ranks=False)
    check_select_index(x, "mod_lt", m, s)
    say(f"  MOD_LT({m}, {s}) {keep}: kept {kept} of {n}")


def test_runs_of_every_length_within_a_chunk():
    """Each 2048-element wavefront chunk keeps its first k elements, k running
    over 0..2048 in a scattered order, so every run length meets every
    alignment of its start in the output (the run writes' head, whole 64-word
    pieces, the optional second half of them and the tail)."""
    chunks = 160
    x = wl.full_int32(0x5EED0E00, chunks * C2).astype(np.int64) & ~1  # all even
    for c in range(chunks):
        k = (c * 613 + 1000) % (C2 + 1)
        x[c * C2: c * C2 + k] |= 1
    x = x.astype(np.int32)
    for n in (x.size, x.size - 777):
        kept = check_compact(x[:n], "odd", ranks=False)
        check_select_index(x[:n], "odd")
        check_compact(x[:n], "odd")
        say(f"  n={n}: kept {kept}")


def f32_input(seed: int, n: int) -> np.ndarray:
    """fp32 values in [-2, 2) with NaN, +-0, +-inf and denormals planted."""
    x = (wl.unit_float32(seed, n) * 4 - 2).astype(np.float32)
    special = np.array([np.nan, 0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 0.5, 1.0, -1.0],
                       np.float32)
    x[:min(n, special.size)] = special[:min(n, special.size)]
    if n > 100:
        x[n // 2: n // 2 + special.size] = special
        x[-3:] = [np.nan, -0.0, 0.25]
    return x


F32_CASES = [("f32_nonzero", 0.0, 0.0), ("f32_gt", 0.5, 0.0), ("f32_lt", -0.25, 0.0),
             ("f32_in", 0.0, 1.0), ("f32_gt", float("nan"), 0.0), ("f32_in", -float("inf"), 0.0)]


def bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint32)


@pytest.mark.parametrize("pred,a,b", F32_CASES)
@pytest.mark.parametrize("n", [1, 7, C2 + 3, 3 * T + 611])
def test_f32_compact_partition_select(pred, a, b, n):
    """fp32 elements, IEEE predicates: bit-exact against the oracle (values move
    bit for bit, so -0.0 and NaN come out as they went in)."""
    x = f32_input(n + 3, n)
    p = ssc.PRED[pred]
    xd = dev(x)
    want, m = oracle.compact_f32(x, p, a, b)
    out = torch.full_like(xd, float("nan"))
    _, cnt, rk = ssc.compact(xd, pred, a, b, out=out, ranks=True)
    assert int(host(cnt)[0]) == m
    assert checks.first_mismatch(bits(host(out)[:m]), bits(want)) == -1
    flags = np.array([oracle.pred_f32(float(v), p, a, b) for v in x[:2000]], np.int32)
    assert checks.first_mismatch(host(rk)[:flags.size], np.cumsum(flags) - flags) == -1
    pw, k = oracle.partition_f32(x, p, a, b)
    pout, kc = ssc.partition(xd, pred, a, b)
    assert int(host(kc)[0]) == k
    assert checks.first_mismatch(bits(host(pout)), bits(pw)) == -1
    iw, mi = oracle.select_index_f32(x, p, a, b)
    idx = torch.full((n,), SENTINEL, dtype=torch.int32, device=DEV)
    _, ic = ssc.select_index(xd, pred, a, b, out=idx)
    assert int(host(ic)[0]) == mi
    o = host(idx)
    assert checks.first_mismatch(o[:mi], iw) == -1 and np.all(o[mi:] == SENTINEL)


def test_f32_compaction_large():
    """2^26 fp32 values, keep 0 <= x < 1 (about a quarter)."""
    x = f32_input(99, 1 << 26)
    want, m = oracle.compact_f32(x, oracle.PRED_F32_IN, 0.0, 1.0)
    out, cnt = ssc.compact(dev(x), "f32_in", 0.0, 1.0)
    assert int(host(cnt)[0]) == m
    assert checks.first_mismatch(bits(host(out)[:m]), bits(want)) == -1


@pytest.mark.parametrize("n", [1, 5, 8191, 8192, 8193, 3 * T + 611, 8192 * 8192 + 77, 10_000_000])
def test_multipass_pipelines_match_the_oracle(n):
    """The multi-launch comparison pipelines (one, two and three levels of tile
    sums) give the oracle's results, like the single pass."""
    x = wl.uniform_below(n + 5, n, 7) - 2
    xd = dev(x)
    want, total = oracle.exclusive_scan_i32(x)
    out, tot = ssc.exclusive_scan_multipass(xd)
    assert checks.first_mismatch(host(out), want) == -1 and int(host(tot)[0]) == total
    y = xd.clone()
    ssc.exclusive_scan_multipass(y, out=y)
    assert checks.first_mismatch(host(y), want) == -1
    surv, m, ranks = oracle.compact_i32(x, oracle.PRED_NONZERO, want_ranks=True)
    o = torch.full_like(xd, SENTINEL)
    _, cnt, rk = ssc.compact_multipass(xd, "nonzero", out=o)
    assert int(host(cnt)[0]) == m
    got = host(o)
    assert checks.first_mismatch(got[:m], surv) == -1 and np.all(got[m:] == SENTINEL)
    assert checks.first_mismatch(host(rk), ranks) == -1


def test_keep_all_is_copy_and_keep_none_writes_nothing():
    x = wl.uniform_below(5, 7 * T + 77, 9) + 1
    out, cnt = ssc.compact(dev(x), "nonzero")
    assert int(host(cnt)[0]) == x.size
    assert checks.first_mismatch(host(out), x) == -1
    check_compact(np.zeros(7 * T + 77, np.int32), "nonzero")   # count 0, out untouched
    check_partition(x, "mod_lt", 100, 0)                        # nothing kept: out == in
    check_partition(x, "nonzero")   # everything kept: each rejected run starts at its region's end


@pytest.mark.parametrize("n", [S - 3, 3 * T + 611, 100_003])
def test_unaligned_arrays_take_the_32bit_path(n):  # noqa: C901
    """Arrays 4-byte but not 16-byte aligned (offset by one element)."""
    x = wl.uniform_below(9, n + 1, 10)
    base = dev(x)
    xs = base[1:]           # 4 bytes past a 256-byte allocation boundary
    assert xs.data_ptr() % 16 == 4
    want, m, want_ranks = oracle.compact_i32(x[1:], oracle.PRED_EVEN, want_ranks=True)
    out_buf = torch.full((n + 1,), SENTINEL, dtype=torch.int32, device=DEV)
    ranks_buf = torch.zeros(n + 1, dtype=torch.int32, device=DEV)
    out, cnt, rk = ssc.compact(xs, "even", out=out_buf[1:], ranks=ranks_buf[1:])
    assert int(host(cnt)[0]) == m
    assert checks.first_mismatch(host(out)[:m], want) == -1
    assert checks.first_mismatch(host(rk), want_ranks) == -1
    pw, k = oracle.partition_i32(x[1:], oracle.PRED_EVEN)
    pout = torch.empty(n + 1, dtype=torch.int32, device=DEV)[1:]
    ssc.partition(xs, "even", out=pout)
    assert checks.first_mismatch(host(pout), pw) == -1
    sw, stot = oracle.exclusive_scan_i32(x[1:])
    sout = torch.empty(n + 1, dtype=torch.int32, device=DEV)[1:]
    _, tot = ssc.exclusive_scan(xs, out=sout)
    assert checks.first_mismatch(host(sout), sw) == -1 and int(host(tot)[0]) == stot
    cp = torch.empty(n + 1, dtype=torch.int32, device=DEV)[1:]
    ssc.copy(xs, cp)
    assert checks.first_mismatch(host(cp), x[1:]) == -1
    iw, mi = oracle.select_index_i32(x[1:], oracle.PRED_EVEN)
    iout = torch.full((n + 1,), SENTINEL, dtype=torch.int32, device=DEV)[1:]
    _, icnt = ssc.select_index(xs, "even", out=iout)
    assert int(host(icnt)[0]) == mi and checks.first_mismatch(host(iout)[:mi], iw) == -1
    inc = torch.empty(n + 1, dtype=torch.int32, device=DEV)[1:]
    ssc.inclusive_scan(xs, out=inc)
    assert checks.first_mismatch(host(inc), oracle.inclusive_scan_i32(x[1:])) == -1


def test_scan_i32_wraps_and_in_place():
    x = wl.full_int32(31337, 9 * T + 5)
    want, total = oracle.exclusive_scan_i32(x)
    xd = dev(x)
    out, tot = ssc.exclusive_scan(xd, out=xd)       # in place
    assert out.data_ptr() == xd.data_ptr()
    assert checks.first_mismatch(host(xd), want) == -1
    assert int(host(tot)[0]) == total


# Tile counts that take each scan launch, and the counts on both sides of
# each switch: at most one tile per compute unit (persistent, one tile each),
# one to two (one workgroup per tile), two to three (persistent, later tiles
# claimed one at a time) and three or more (persistent, second and third
# tiles claimed together). MI355X has 256 compute units.
SCAN_TILE_COUNTS = [33, 256, 257, 326, 512, 513, 700, 767, 768, 1500]


@pytest.mark.parametrize("tiles", SCAN_TILE_COUNTS)
def test_scan_paths_by_tile_count(tiles):
    """Exclusive and inclusive int32 (bit-exact, also in place and from
    unaligned arrays) and fp32 exclusive (1e-5) at each launch shape, with a
    ragged last tile."""
    n = (tiles - 1) * T + 611
    x = wl.full_int32(0x5CA9 + tiles, n)
    xd = dev(x)
    want, total = oracle.exclusive_scan_i32(x)
    out, tot = ssc.exclusive_scan(xd)
    assert checks.first_mismatch(host(out), want) == -1 and int(host(tot)[0]) == total
    check_inclusive_i32(x, xd=xd)
    y = xd.clone()
    ssc.exclusive_scan(y, out=y)
    assert checks.first_mismatch(host(y), want) == -1
    base = torch.empty(n + 1, dtype=torch.int32, device=DEV)
    base[1:] = xd
    uo = torch.empty(n + 1, dtype=torch.int32, device=DEV)[1:]
    assert base[1:].data_ptr() % 16 == 4
    _, tot = ssc.exclusive_scan(base[1:], out=uo)
    assert checks.first_mismatch(host(uo), want) == -1 and int(host(tot)[0]) == total
    del out, y, base, uo
    check_scan_f32(wl.unit_float32(0x5CAF + tiles, n))


@pytest.mark.parametrize("tiles", [256, 257, 767, 768])
def test_compaction_paths_by_tile_count(tiles):
    """The persistent compaction kernel on both sides of its switches: one
    tile per workgroup or more, and the second and third tiles claimed one at
    a time (below three per workgroup) or together. Compaction with ranks,
    partition and selection, with a ragged last tile."""
    n = (tiles - 1) * T + 611
    x = wl.full_int32(0xC0A7 + tiles, n)
    xd = dev(x)
    check_compact(x, "odd", xd=xd)
    check_compact(x, "mod_lt", 100, 50, xd=xd, ranks=False)
    check_partition(x, "even", xd=xd)
    check_select_index(x, "mod_lt", 100, 1, xd=xd)


def test_repeated_runs_are_identical():
    """The look-back must give the same answer whatever order tiles finish in:
    100 compactions and 100 scans of 1,500 tiles (several per workgroup, every
    claim path) on one scratch, each compared with the oracle."""
    n = 1499 * T + 17
    x = wl.uniform_below(4242, n, 3)
    want, m = oracle.compact_i32(x, oracle.PRED_NONZERO)
    xd = dev(x)
    scratch = ssc.new_scratch(x.size, xd.device)
    out = torch.empty_like(xd)
    cnt = torch.empty(1, dtype=torch.int32, device=DEV)
    wd = dev(want)
    for it in range(100):
        ssc.compact(xd, "nonzero", out=out, count=cnt, scratch=scratch)
        assert int(host(cnt)[0]) == m, it
        assert torch.equal(out[:m], wd), it
    sw, _ = oracle.exclusive_scan_i32(x)
    swd = dev(sw)
    sout = torch.empty_like(xd)
    for it in range(100):
        ssc.exclusive_scan(xd, out=sout, scratch=scratch)
        assert torch.equal(sout, swd), it
    assert not ssc.timed_out(scratch)


@pytest.mark.parametrize("shift_words", [4, 12])
def test_outputs_that_start_inside_a_cache_line(shift_words):
    """Runs are stored by 128-byte line: the partial first and last lines
    with the default policy, whole lines nontemporal. An output array that is
    16-byte aligned (the 128-bit path) but starts 16 or 48 bytes into a line
    puts every run boundary at another offset. Compaction, partition (every
    slot written) and selection must still match the oracle exactly and
    leave everything outside their output untouched."""
    n = 3 * T + 2 * C2 + 17
    x = wl.uniform_below(0x5EED0909 + shift_words, n, 3)
    xd = dev(x)
    base = torch.full((n + 64,), SENTINEL, dtype=torch.int32, device=DEV)
    out = base[shift_words:shift_words + n]
    assert out.data_ptr() % 16 == 0 and out.data_ptr() % 128 != 0

    def check(want, m, what):
        h = host(base)
        assert checks.first_mismatch(h[shift_words:shift_words + m], want) == -1, what
        assert (h[:shift_words] == SENTINEL).all(), what
        assert (h[shift_words + m:] == SENTINEL).all(), what

    want, m = oracle.compact_i32(x, oracle.PRED_NONZERO)
    _, cnt = ssc.compact(xd, "nonzero", out=out)
    assert int(host(cnt)[0]) == m
    check(want, m, "compact")
    base.fill_(SENTINEL)
    pw, k = oracle.partition_i32(x, oracle.PRED_EVEN)
    _, kc = ssc.partition(xd, "even", out=out)
    assert int(host(kc)[0]) == k
    check(pw, n, "partition")
    base.fill_(SENTINEL)
    iw, mi = oracle.select_index_i32(x, oracle.PRED_NONZERO)
    _, ci = ssc.select_index(xd, "nonzero", out=out)
    assert int(host(ci)[0]) == mi
    check(iw, mi, "select")


def test_look_back_wait_is_bounded_and_reported():
    """A descriptor that is never published must not keep the kernel
    running: the host starts a fresh scratch's tile counter at 1, so tile 0
    is never claimed and tile 1's look-back waits on it. The wait gives up
    after its fixed number of polls (about a second), the kernel finishes
    normally and word 2 of the scratch reports it; a zeroed scratch then
    serves a correct call again."""
    import time
    x = wl.uniform_below(77, 4 * T, 3)
    want, m = oracle.compact_i32(x, oracle.PRED_NONZERO)
    xd = dev(x)
    scratch = ssc.new_scratch(x.size, xd.device)
    scratch[0:8].view(torch.int64)[0] = 1  # {epoch 0 | next tile 1}
    torch.cuda.synchronize()
    t0 = time.time()
    ssc.compact(xd, "nonzero", scratch=scratch)
    torch.cuda.synchronize()
    say(f"  forced look-back time-out: call finished after {time.time() - t0:.2f} s")
    assert int(host(scratch[8:12].view(torch.int32))[0]) == 1
    scratch.zero_()
    out, cnt = ssc.compact(xd, "nonzero", scratch=scratch)
    assert int(host(cnt)[0]) == m
    assert checks.first_mismatch(host(out)[:m], want) == -1
    assert int(host(scratch[8:12].view(torch.int32))[0]) == 0


def test_one_scratch_across_sizes_and_ops():
    """One scratch buffer serves many calls of different sizes and kinds in a
    row: the epoch tags keep descriptors of earlier calls from being read."""
    big = wl.uniform_below(123, 40 * T + 7, 5)
    small = wl.uniform_below(321, 3 * T + 1, 5)
    scratch = ssc.new_scratch(big.size, torch.device(DEV))
    plan = [big, small, big, small[:100], big, small, big[: T + 1], big]
    for it, x in enumerate(plan):
        xd = dev(x)
        want, m = oracle.compact_i32(x, oracle.PRED_NONZERO)
        out, cnt = ssc.compact(xd, "nonzero", scratch=scratch)
        assert int(host(cnt)[0]) == m, it
        assert checks.first_mismatch(host(out)[:m], want) == -1, it
        sw, stot = oracle.exclusive_scan_i32(x)
        sout, tot = ssc.exclusive_scan(xd, scratch=scratch)
        assert checks.first_mismatch(host(sout), sw) == -1, it
        pw, k = oracle.partition_i32(x, oracle.PRED_ODD)
        pout, kc = ssc.partition(xd, "odd", scratch=scratch)
        assert int(host(kc)[0]) == k and checks.first_mismatch(host(pout), pw) == -1, it
        c = ssc.count_if(xd, "even", scratch=scratch)
        assert int(host(c)[0]) == oracle.count(x, oracle.PRED_EVEN), it
    assert int(host(scratch[8:12].view(torch.int32))[0]) == 0


def test_scratch_init_zero_fills():
    scratch = torch.full((ssc.scratch_bytes(5 * T),), 0x5A, dtype=torch.uint8, device=DEV)
    rc = ssc.lib().ssc_scratch_init(scratch.data_ptr(), scratch.numel(),
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    assert int(host(scratch).astype(np.int64).sum()) == 0
    x = wl.uniform_below(77, 5 * T, 3)
    want, m = oracle.compact_i32(x, oracle.PRED_NONZERO)
    out, cnt = ssc.compact(dev(x), "nonzero", scratch=scratch)
    assert int(host(cnt)[0]) == m
    assert checks.first_mismatch(host(out)[:m], want) == -1


def test_runs_on_a_side_stream():
    x = wl.uniform_below(99, 123_457, 4)
    want, m = oracle.compact_i32(x, oracle.PRED_NONZERO)
    xd = dev(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out, cnt = ssc.compact(xd, "nonzero")
    s.synchronize()
    assert int(cnt.cpu()[0]) == m
    assert checks.first_mismatch(out.cpu().numpy()[:m], want) == -1


def test_concurrent_calls_on_three_streams():
    """Three calls of the persistent kernel in flight at once on three streams
    (each with its own scratch), repeated without host synchronization. One
    workgroup fills a compute unit's LDS, so the calls' grids share the GPU
    and none is fully resident from the start; tiles are numbered by claims
    of running workgroups only, so each call still finishes with the
    oracle's result, and every call leaves its counter reset for the next."""
    n1, n2, n3 = (1 << 22) + 17, (1 << 21) + 5, 3 * T + 611
    x1 = wl.full_int32(501, n1)
    k2 = wl.uniform_below(502, n2, 5)
    v2 = wl.full_int32(503, n2)
    x3 = wl.full_int32(504, n3)
    w1, m1 = oracle.compact_i32(x1, oracle.PRED_ODD)
    wk, wv, m2 = oracle.compact_kv(k2, v2, oracle.PRED_NONZERO)
    w3, k3 = oracle.partition_i32(x3, oracle.PRED_EVEN)
    d1, dk, dv, d3 = dev(x1), dev(k2), dev(v2), dev(x3)
    sc = [ssc.new_scratch(n, DEV) for n in (n1, n2, n3)]
    streams = [torch.cuda.Stream() for _ in range(3)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    outs = None
    for _ in range(4):
        with torch.cuda.stream(streams[0]):
            o1 = ssc.compact(d1, "odd", scratch=sc[0])
        with torch.cuda.stream(streams[1]):
            o2 = ssc.compact_kv(dk, dv, "nonzero", scratch=sc[1])
        with torch.cuda.stream(streams[2]):
            o3 = ssc.partition(d3, "even", scratch=sc[2])
        outs = (o1, o2, o3)
    for st in streams:
        st.synchronize()
    (o1, c1), (ok, ov, c2), (o3, c3) = outs
    assert int(c1.cpu()[0]) == m1 and int(c2.cpu()[0]) == m2 and int(c3.cpu()[0]) == k3
    assert checks.first_mismatch(o1.cpu().numpy()[:m1], w1) == -1
    assert checks.first_mismatch(ok.cpu().numpy()[:m2], wk) == -1
    assert checks.first_mismatch(ov.cpu().numpy()[:m2], wv) == -1
    assert checks.first_mismatch(o3.cpu().numpy(), w3) == -1
    # no look-back gave up waiting
    for s_ in sc:
        assert int(s_[8:12].view(torch.int32).cpu()[0]) == 0


def test_graph_capture_replays_match_the_oracle():
    """The calls are one launch each (partition: two) with no memset and no
    allocation, and the claim counter's epoch lives in the scratch, so they
    can be captured in a HIP graph: each replay, with eager work and host
    synchronization between replays, gives the oracle's result."""
    n = 7 * T + 123
    x = wl.full_int32(505, n)
    want, m = oracle.compact_i32(x, oracle.PRED_ODD)
    pwant, k = oracle.partition_i32(x, oracle.PRED_EVEN)
    swant, stot = oracle.exclusive_scan_i32(x)
    xd = dev(x)
    out = torch.empty_like(xd)
    pout = torch.empty_like(xd)
    sout = torch.empty_like(xd)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    pcnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    tot = torch.zeros(1, dtype=torch.int32, device=DEV)
    sc = [ssc.new_scratch(n, DEV) for _ in range(3)]

    def calls():
        ssc.compact(xd, "odd", out=out, count=cnt, scratch=sc[0])
        ssc.partition(xd, "even", out=pout, count=pcnt, scratch=sc[1])
        ssc.exclusive_scan(xd, out=sout, total=tot, scratch=sc[2])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for _ in range(4):
        out.fill_(SENTINEL)
        pout.fill_(SENTINEL)
        sout.fill_(SENTINEL)
        cnt.zero_()
        pcnt.zero_()
        tot.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(cnt.cpu()[0]) == m and int(pcnt.cpu()[0]) == k and int(tot.cpu()[0]) == stot
        o = out.cpu().numpy()
        assert checks.first_mismatch(o[:m], want) == -1 and np.all(o[m:] == SENTINEL)
        assert checks.first_mismatch(pout.cpu().numpy(), pwant) == -1
        assert checks.first_mismatch(sout.cpu().numpy(), swant) == -1
    del g


def test_prepared_call_repeats_the_same_library_call():
    x = wl.full_int32(91, 3 * T + 5)
    want, m = oracle.compact_i32(x, oracle.PRED_ODD)
    xd = dev(x)
    out = torch.full_like(xd, SENTINEL)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    run = ssc.prepared(ssc.compact, xd, "odd", out=out, count=cnt)
    # the scratch compact() allocated for itself must outlive the call: fresh
    # allocations of that size, filled with ones, would otherwise land on it
    churn = [torch.full((ssc.scratch_bytes(x.size) + 64 * i,), 255, dtype=torch.uint8, device=DEV)
             for i in range(16)]
    for _ in range(3):
        out.fill_(SENTINEL)
        cnt.zero_()
        got_out, got_cnt = run()
        assert got_out is out and got_cnt is cnt
        assert int(host(cnt)[0]) == m
        o = host(out)
        assert checks.first_mismatch(o[:m], want) == -1 and np.all(o[m:] == SENTINEL)
    del churn


def test_argument_errors_raise_on_gpu():
    x = torch.zeros(1000, dtype=torch.int32, device=DEV)
    with pytest.raises(ssc.SSCError):
        ssc.compact(x, "bit_set", 40)
    with pytest.raises(ssc.SSCError):
        ssc.partition(x, "even", out=x)
    with pytest.raises(ValueError):
        ssc.compact(x, "odd", scratch=torch.empty(8, dtype=torch.uint8, device=DEV))


@pytest.mark.gpu
def test_binding_checks_caller_tensors_before_launch():
    """Every tensor a caller passes is checked in the binding (GPU, device,
    contiguity, dtype, size) before its pointer reaches the library, so an
    undersized output or a host-side scratch raises instead of being written
    past its end or handed to device atomics; the sentinel output stays."""
    n = 5000
    x = torch.arange(n, dtype=torch.int32, device=DEV)
    sentinel = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    short = torch.full((n - 1,), -7, dtype=torch.int32, device=DEV)
    sc = ssc.new_scratch(n, DEV)
    cases = [
        (ValueError, lambda: ssc.compact(x, "odd", out=short)),
        (ValueError, lambda: ssc.compact(x, "odd", out=sentinel, ranks=short)),
        (ValueError, lambda: ssc.compact(x, "odd", out=sentinel,
                                         scratch=torch.zeros(sc.numel(), dtype=torch.uint8))),
        (TypeError, lambda: ssc.compact(x, "odd", out=sentinel, scratch=sc.view(torch.int32))),
        (TypeError, lambda: ssc.compact(x, "odd", out=sentinel.float())),
        (ValueError, lambda: ssc.compact(x, "odd", out=sentinel,
                                         count=torch.zeros(0, dtype=torch.int32, device=DEV))),
        (ValueError, lambda: ssc.compact(x, "odd", out=sentinel,
                                         count=torch.zeros(1, dtype=torch.int32))),
        (ValueError, lambda: ssc.partition(x, "even", out=short)),
        (ValueError, lambda: ssc.select_index(x, "odd", out=short)),
        (ValueError, lambda: ssc.exclusive_scan(x, out=short)),
        (TypeError, lambda: ssc.exclusive_scan(x, total=torch.zeros(1, dtype=torch.int64, device=DEV))),
        (ValueError, lambda: ssc.exclusive_scan(x, out=torch.zeros(2 * n, dtype=torch.int32, device=DEV)[::2])),
        (ValueError, lambda: ssc.radix_sort(x, out=sentinel, tmp=short)),
        (ValueError, lambda: ssc.compact_atomic(x, "odd", out=short)),
        (ValueError, lambda: ssc.compact_flags(x, (x & 1).bool(), out=short)),
        (ValueError, lambda: ssc.select_flags((x & 1).bool(), out=short)),
        (ValueError, lambda: ssc.compact_kv(x, x, "odd", keys_out=sentinel, vals_out=short)),
        (ValueError, lambda: ssc.copy(x, out=short)),
        (ValueError, lambda: ssc.scatter(x, short, "odd", out=sentinel)),
    ]
    for err, call in cases:
        with pytest.raises(err):
            call()
    torch.cuda.synchronize()
    assert bool((sentinel == -7).all()) and bool((short == -7).all())


@pytest.mark.gpu
def test_mark_and_scatter_steps_match_the_oracle():
    """The multi-launch compaction's separate steps: mark writes the 0/1
    flags, and scatter with their exclusive scan gives the ordered survivors
    and the count."""
    x_np = wl.full_int32(0x5EED0A11, 3 * 30720 + 77)
    x = torch.from_numpy(x_np).to(DEV)
    flags = ssc.mark(x, "mod_lt", 10, 3)
    want_flags = oracle.flags(x_np, oracle.PRED_MOD_LT, 10, 3)
    assert np.array_equal(flags.cpu().numpy(), want_flags.astype(np.int32))
    ranks, _ = ssc.exclusive_scan(flags)
    out = torch.full_like(x, -7)
    out, cnt = ssc.scatter(x, ranks, "mod_lt", 10, 3, out=out)
    want, m = oracle.compact_i32(x_np, oracle.PRED_MOD_LT, 10, 3)
    torch.cuda.synchronize()
    assert int(cnt.item()) == m
    assert np.array_equal(out[:m].cpu().numpy(), want)
    assert bool((out[m:] == -7).all())
