"""Parity of the HIP path with the CPU oracle for the other element formats of
the persistent compaction kernel: a caller's predicate as flag bytes
(compaction and selection), key-value pairs, and 64-bit elements.

Everything is integer or bit-moving work, so results must match bit for bit,
and nothing past count may be written. Sizes straddle the wavefront chunks
(2048 elements for flag bytes, 1024 for pairs and 64-bit elements), the tiles
(15 chunks), odd byte counts of the flag array, and more tiles than the
kernel has workgroups. The 32-bit path (arrays not 16-byte aligned) is run
through views that start one element in.
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

DEV = "cuda"
SENTINEL = -123456789
SENT64 = -0x0123456789ABCDEF
TF = 15 * 2048   # elements per tile, flag bytes
TH = 15 * 1024   # elements per tile, pairs and 64-bit elements

FLAG_N = [1, 2, 3, 4, 5, 63, 64, 65, 255, 257, 2047, 2048, 2049, TF - 1, TF, TF + 1,
          3 * TF + 611, 300 * TF + 17]
HALF_N = [1, 2, 3, 7, 1023, 1024, 1025, 2049, TH - 1, TH, TH + 1, 2 * TH + 3, 7 * TH + 611,
          300 * TH + 29]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def shifted(a: np.ndarray) -> torch.Tensor:
    """A device copy of a that starts one element into its allocation (so it
    is 4- or 8-byte aligned but not 16-byte aligned)."""
    big = torch.empty(a.size + 1, dtype=torch.from_numpy(a[:0].copy()).dtype, device=DEV)
    v = big[1:]
    v.copy_(torch.from_numpy(np.ascontiguousarray(a)))
    assert v.data_ptr() % 16 != 0
    return v


def check_flags(x: np.ndarray, f: np.ndarray, xd=None, fd=None):
    want, m = oracle.compact_flags(x, f)
    xd = dev(x) if xd is None else xd
    fd = dev(f) if fd is None else fd
    out = torch.full((x.size,), SENTINEL, dtype=torch.int32, device=DEV).view(xd.dtype)
    _, cnt = ssc.compact_flags(xd, fd, out=out)
    assert int(host(cnt)[0]) == m
    o = host(out).view(np.uint32)
    assert checks.first_mismatch(o[:m], want.view(np.uint32)) == -1
    assert np.all(o[m:].view(np.int32) == SENTINEL), "compaction wrote past count"
    wi, mi = oracle.select_flags(f)
    idx = torch.full((x.size,), SENTINEL, dtype=torch.int32, device=DEV)
    _, c2 = ssc.select_flags(fd, out=idx)
    assert int(host(c2)[0]) == mi == m
    oi = host(idx)
    assert checks.first_mismatch(oi[:m], wi) == -1
    assert np.all(oi[m:] == SENTINEL), "selection wrote past count"
    return m


@pytest.mark.parametrize("n", FLAG_N)
def test_flag_bytes_compaction_and_selection(n):
    say(f"  flags n={n}")
    x = wl.full_int32(300 + n, n)
    for keep in (0, 37, 100):
        check_flags(x, wl.flag_bytes(400 + n + keep, n, keep))


def test_flag_bytes_float_values_bool_mask_and_unaligned_values():
    n = 5 * TF + 1237
    x = wl.unit_float32(17, n) * 2 - 1
    x[:4] = [np.nan, -0.0, np.inf, 1e-45]
    f = wl.flag_bytes(18, n, 50)
    f[:4] = [255, 1, 0, 2]
    check_flags(x, f)
    # a torch.bool mask is a flag-byte array
    xi = wl.full_int32(19, n)
    mask = xi % 3 == 0
    want, m = oracle.compact_flags(xi, mask.astype(np.uint8))
    out, cnt = ssc.compact_flags(dev(xi), dev(mask))
    assert int(host(cnt)[0]) == m
    assert checks.first_mismatch(host(out)[:m], want) == -1
    # values not 16-byte aligned take the 32-bit loads
    check_flags(xi, f, xd=shifted(xi))


def test_flag_bytes_full_size():
    """2^28 int32 values with a 50% flag array: the headline's size."""
    n = wl.N_HEADLINE
    say("  generating 2^28 values and flags ...")
    x = wl.headline_input()
    f = wl.flag_bytes(0x5EED0104, n, 50)
    m = check_flags(x, f)
    say(f"  kept {m} of {n}")


# Selection by flag bytes from a 16-byte aligned array takes its own kernel:
# 4096 flags per data wavefront (four 128-bit loads per lane), 61,440 per
# tile, written in rounds of 2048. Sizes around a round, its chunk and tile,
# byte counts that end inside a dword, and tile counts on both sides of the
# claim paths (256 compute units; the second and third tiles are claimed
# together from 768 tiles).
CH = 4096
TS = 15 * CH
SEL_FLAG_N = [2047, 2048, 2049, CH - 1, CH, CH + 1, CH + 3, 2 * CH + 7, TS - 1, TS, TS + 1, TS + 3,
              3 * TS + 611, 256 * TS, 256 * TS + 1, 257 * TS + 13, 767 * TS + 9, 768 * TS,
              800 * TS + 5]


@pytest.mark.parametrize("n", SEL_FLAG_N)
def test_selection_by_flag_bytes_large_tiles(n):
    say(f"  selection by flags n={n}")
    for keep in (0, 1, 50, 100):
        f = wl.flag_bytes(500 + n + keep, n, keep)
        want, m = oracle.select_flags(f)
        fd = dev(f)
        assert fd.data_ptr() % 16 == 0
        idx = torch.full((n,), SENTINEL, dtype=torch.int32, device=DEV)
        _, cnt = ssc.select_flags(fd, out=idx)
        assert int(host(cnt)[0]) == m, (n, keep)
        o = host(idx)
        assert checks.first_mismatch(o[:m], want) == -1, (n, keep)
        assert np.all(o[m:] == SENTINEL), "selection wrote past count"
        if n <= 3 * TS + 611:
            # 4-byte but not 16-byte aligned flags keep the compaction kernel's format
            big = torch.zeros(n + 4, dtype=torch.uint8, device=DEV)
            fu = big[4:]
            fu.copy_(fd)
            assert fu.data_ptr() % 16 == 4
            idx.fill_(SENTINEL)
            _, cnt = ssc.select_flags(fu, out=idx)
            assert int(host(cnt)[0]) == m
            o = host(idx)
            assert checks.first_mismatch(o[:m], want) == -1 and np.all(o[m:] == SENTINEL)


def test_selection_by_flag_bytes_every_byte_value():
    """Every byte value 0..255 at every byte offset within the 16-byte words
    the large-tile kernel loads (block b of 256 flags is 0..255 rotated by b),
    repeated past one chunk; nonzero means kept, whatever the bits."""
    i = np.arange(256 * 16 * 3, dtype=np.int64)
    f = ((i % 256 + (i // 256) % 16) % 256).astype(np.uint8)
    want, m = oracle.select_flags(f)
    assert m == f.size - f.size // 256
    fd = dev(f)
    assert fd.data_ptr() % 16 == 0
    idx, cnt = ssc.select_flags(fd)
    assert int(host(cnt)[0]) == m
    assert checks.first_mismatch(host(idx)[:m], want) == -1
    x = wl.full_int32(0xB17E, f.size)
    check_flags(x, f)


def check_kv(keys: np.ndarray, vals: np.ndarray, pred, a=0, b=0, kd=None, vd=None):
    p = ssc.PRED[pred] if isinstance(pred, str) else pred
    wk, wv, m = oracle.compact_kv(keys, vals, p, a, b)
    kd = dev(keys) if kd is None else kd
    vd = dev(vals) if vd is None else vd
    ko = torch.full((keys.size,), SENTINEL, dtype=torch.int32, device=DEV).view(kd.dtype)
    vo = torch.full((keys.size,), SENTINEL, dtype=torch.int32, device=DEV).view(vd.dtype)
    _, _, cnt = ssc.compact_kv(kd, vd, p, a, b, keys_out=ko, vals_out=vo)
    assert int(host(cnt)[0]) == m, (pred, a, b)
    k, v = host(ko).view(np.uint32), host(vo).view(np.uint32)
    assert checks.first_mismatch(k[:m], wk.view(np.uint32)) == -1
    assert checks.first_mismatch(v[:m], wv.view(np.uint32)) == -1
    assert np.all(k[m:].view(np.int32) == SENTINEL) and np.all(v[m:].view(np.int32) == SENTINEL)
    return m


KV_CASES = [("nonzero", 0, 0), ("odd", 0, 0), ("even", 0, 0), ("bit_set", 31, 0),
            ("bit_clear", 3, 0), ("mod_lt", 100, 50), ("mod_lt", 7, 0)]


@pytest.mark.parametrize("n", HALF_N)
def test_key_value_pairs_edge_sizes(n):
    say(f"  pairs n={n}")
    keys = wl.uniform_below(500 + n, n, 7) - 3
    vals = (np.arange(n, dtype=np.uint32) * np.uint32(2654435761)).view(np.int32)
    check_kv(keys, vals, "nonzero")
    check_kv(keys, vals, "odd")


@pytest.mark.parametrize("pred,a,b", KV_CASES)
def test_key_value_every_predicate(pred, a, b):
    n = 3 * TH + 611
    keys = wl.full_int32(600, n)
    keys[:6] = [0, -1, 1, -2147483648, 2147483647, -100]
    vals = wl.unit_float32(601, n)
    check_kv(keys, vals, pred, a, b)


def test_key_value_float_keys_and_unaligned():
    n = 9 * TH + 77
    fk = wl.unit_float32(602, n) * 4 - 2
    fk[:5] = [np.nan, -0.0, 0.0, np.inf, -np.inf]
    vals = np.arange(n, dtype=np.int32)
    with np.errstate(invalid="ignore"):
        for pred, a, b in [("f32_nonzero", 0.0, 0.0), ("f32_gt", 0.5, 0.0), ("f32_lt", -1.0, 0.0),
                           ("f32_in", -0.5, 0.5)]:
            check_kv(fk, vals, pred, a, b)
    keys = wl.full_int32(603, n)
    check_kv(keys, vals, "odd", kd=shifted(keys), vd=shifted(vals))
    check_kv(keys, vals, "even", vd=shifted(vals))


def test_key_value_full_size():
    """2^27 int32 keys (odd kept) with 2^27 values: 1 GiB in, as the headline."""
    n = wl.N_HEADLINE // 2
    say("  generating 2^27 pairs ...")
    keys = wl.headline_input(n)
    vals = wl.full_int32(0x5EED0105, n)
    m = check_kv(keys, vals, "odd")
    say(f"  kept {m} of {n}")


def check_i64(x: np.ndarray, pred, bit=0, xd=None):
    p = ssc.PRED[pred] if isinstance(pred, str) else pred
    want, m = oracle.compact_i64(x, p, bit)
    xd = dev(x) if xd is None else xd
    out = torch.full((x.size,), SENT64, dtype=torch.int64, device=DEV)
    _, cnt = ssc.compact(xd, p, bit, out=out)
    assert int(host(cnt)[0]) == m, (pred, bit)
    o = host(out)
    assert checks.first_mismatch(o[:m], want) == -1
    assert np.all(o[m:] == SENT64), "compaction wrote past count"
    wi, mi = oracle.select_index_i64(x, p, bit)
    idx = torch.full((x.size,), SENTINEL, dtype=torch.int32, device=DEV)
    _, c2 = ssc.select_index(xd, p, bit, out=idx)
    assert int(host(c2)[0]) == mi
    oi = host(idx)
    assert checks.first_mismatch(oi[:mi], wi) == -1
    assert np.all(oi[mi:] == SENTINEL), "selection wrote past count"
    return m


I64_CASES = [("nonzero", 0), ("odd", 0), ("even", 0), ("bit_set", 0), ("bit_set", 31),
             ("bit_set", 32), ("bit_set", 63), ("bit_clear", 33), ("bit_clear", 62)]


@pytest.mark.parametrize("n", HALF_N)
def test_int64_edge_sizes(n):
    say(f"  int64 n={n}")
    x = wl.full_int64(700 + n, n)
    check_i64(x, "odd")
    check_i64(x, "bit_set", 40)


@pytest.mark.parametrize("pred,bit", I64_CASES)
def test_int64_every_predicate(pred, bit):
    n = 3 * TH + 611
    x = wl.full_int64(701, n)
    x[:6] = [0, -1, 1, -2**63, 2**63 - 1, 2**32]
    x[6:12] = 0  # some zeros for nonzero
    check_i64(x, pred, bit)


def test_int64_unaligned_takes_64bit_loads_and_full_size():
    n = 5 * TH + 333
    x = wl.full_int64(702, n)
    check_i64(x, "odd", xd=shifted(x))
    check_i64(x, "bit_clear", 63, xd=shifted(x))
    n = wl.N_HEADLINE // 2
    say("  generating 2^27 int64 ...")
    x = wl.full_int64(0x5EED0106, n)
    m = check_i64(x, "odd")
    say(f"  kept {m} of {n}")


def test_other_formats_empty_and_errors():
    z = torch.empty(0, dtype=torch.int32, device=DEV)
    _, cnt = ssc.compact_flags(z, torch.empty(0, dtype=torch.bool, device=DEV))
    assert int(host(cnt)[0]) == 0
    _, _, cnt = ssc.compact_kv(z, z.clone(), "odd")
    assert int(host(cnt)[0]) == 0
    _, cnt = ssc.compact(torch.empty(0, dtype=torch.int64, device=DEV), "odd")
    assert int(host(cnt)[0]) == 0
    x64 = torch.zeros(10, dtype=torch.int64, device=DEV)
    with pytest.raises(ssc.SSCError):
        ssc.compact(x64, "bit_set", 64)
    with pytest.raises(ssc.SSCError):
        ssc.compact(x64, "mod_lt", 100, 5)
    with pytest.raises(ssc.SSCError):  # flags not 4-byte aligned
        big = torch.ones(20, dtype=torch.uint8, device=DEV)
        ssc.compact_flags(torch.zeros(10, dtype=torch.int32, device=DEV), big[1:11])


def test_prepared_calls_of_every_format_survive_allocation_churn():
    """A prepared call keeps the scratch its op allocated for itself: after
    fresh allocations (which would reuse freed memory) every replay still
    gives the oracle's result. Timing loops depend on this."""
    n = 4 * TH + 99
    keys = wl.full_int32(800, n)
    vals = wl.full_int32(801, n)
    f = wl.flag_bytes(802, n, 40)
    x64 = wl.full_int64(803, n)
    kd, vd, fd, xd64 = dev(keys), dev(vals), dev(f), dev(x64)
    wk, wv, mk = oracle.compact_kv(keys, vals, oracle.PRED_ODD)
    wf, mf = oracle.compact_flags(keys, f)
    wi, mi = oracle.select_flags(f)
    w64, m64 = oracle.compact_i64(x64, oracle.PRED_ODD)
    runs = [
        (ssc.prepared(ssc.compact_kv, kd, vd, "odd"), lambda r: (r[2], [(r[0], wk), (r[1], wv)], mk)),
        (ssc.prepared(ssc.compact_flags, kd, fd), lambda r: (r[1], [(r[0], wf)], mf)),
        (ssc.prepared(ssc.select_flags, fd), lambda r: (r[1], [(r[0], wi)], mi)),
        (ssc.prepared(ssc.compact, xd64, "odd"), lambda r: (r[1], [(r[0], w64)], m64)),
    ]
    churn = [torch.full((ssc.scratch_bytes(n) + 256 * i,), 255, dtype=torch.uint8, device=DEV)
             for i in range(32)]
    for _ in range(3):
        for run, unpack in runs:
            cnt, outs, m = unpack(run())
            assert int(host(cnt)[0]) == m
            for got, want in outs:
                assert checks.first_mismatch(host(got)[:m], want) == -1
    del churn
