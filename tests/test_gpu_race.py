"""Parity under stress: the same calls through the library's two test builds.

- libssc_perturb.so (the sources compiled with -DSSC_PERTURB) pauses every
  tile claim, descriptor publication, data-wavefront arrival and look-back
  poll for 0 to 7 x 1024 clocks chosen by a hash of the tile, workgroup or
  poll count, so workgroups claim, publish and finish in orders the library
  proper rarely shows.
- libssc_stress.so (-DSSC_STRESS_TILES) gives the persistent kernels tiles
  eight times smaller (3840 elements), so every call makes eight times the
  claims, descriptors and look-backs, and look-backs walk longer windows.

Every result must still match the oracle exactly (fp32 scans within 1e-5),
repeated calls must agree, and no look-back wait may give up.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import scan_stream_compaction_amd as ssc
from scan_stream_compaction_amd import workloads as wl
from tests import checks

pytestmark = [pytest.mark.gpu]

T = 30720
SENTINEL = -123456789


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.fixture(scope="module", params=[ssc.PERTURB_LIB_PATH, ssc.STRESS_LIB_PATH],
                ids=["perturbed", "small_tiles"])
def perturbed(request):
    if not os.path.exists(request.param):
        pytest.skip(f"{os.path.basename(request.param)} not built (python -m scan_stream_compaction_amd.build)")
    with ssc.using_library(request.param) as L:
        yield L


def test_stress_build_has_small_tiles():
    if not os.path.exists(ssc.STRESS_LIB_PATH):
        pytest.skip("libssc_stress.so not built")
    with ssc.using_library(ssc.STRESS_LIB_PATH):
        assert ssc.tile_elems() == 3840
        n = 5 * 3840 + 17
        x = wl.full_int32(0x7AC6, n)
        want, m = oracle.compact_i32(x, oracle.PRED_ODD, 0, 0)
        out, cnt = ssc.compact(dev(x), "odd")
        assert int(host(cnt)[0]) == m and checks.first_mismatch(host(out)[:m], want) == -1


@pytest.mark.parametrize("tiles", [33, 700, 1500])
def test_compaction_family_under_perturbation(perturbed, tiles):
    n = (tiles - 1) * T + 611
    x = wl.full_int32(0x7AC3 + tiles, n)
    xd = dev(x)
    scratch = ssc.new_scratch(n, xd.device)
    for pred, pa, pb in (("odd", 0, 0), ("mod_lt", 100, 1), ("mod_lt", 100, 99)):
        p = ssc.PRED[pred]
        want, m, want_ranks = oracle.compact_i32(x, p, pa, pb, want_ranks=True)
        wd, wr = dev(want), dev(want_ranks)
        out = torch.empty_like(xd)
        for rep in range(3):
            out.fill_(SENTINEL)
            _, cnt, rk = ssc.compact(xd, p, pa, pb, out=out, ranks=True, scratch=scratch)
            assert int(host(cnt)[0]) == m, (pred, pb, rep)
            assert torch.equal(out[:m], wd), (pred, pb, rep)
            assert bool((out[m:] == SENTINEL).all()), (pred, pb, rep)
            assert torch.equal(rk, wr), (pred, pb, rep)
    pw, k = oracle.partition_i32(x, oracle.PRED_EVEN)
    pout, pk = ssc.partition(xd, "even", scratch=scratch)
    assert int(host(pk)[0]) == k and checks.first_mismatch(host(pout), pw) == -1
    iw, mi = oracle.select_index_i32(x, oracle.PRED_ODD)
    idx, icnt = ssc.select_index(xd, "odd", scratch=scratch)
    assert int(host(icnt)[0]) == mi and checks.first_mismatch(host(idx)[:mi], iw) == -1
    f = wl.flag_bytes(0x7AC4 + tiles, n, 50)
    fw, mf = oracle.select_flags(f)
    fidx, fcnt = ssc.select_flags(dev(f), scratch=scratch)
    assert int(host(fcnt)[0]) == mf and checks.first_mismatch(host(fidx)[:mf], fw) == -1
    assert not ssc.timed_out(scratch)


@pytest.mark.parametrize("tiles", [33, 326, 700, 1500])
def test_scans_under_perturbation(perturbed, tiles):
    n = (tiles - 1) * T + 611
    x = wl.full_int32(0x5CA7 + tiles, n)
    xd = dev(x)
    scratch = ssc.new_scratch(n, xd.device)
    want, total = oracle.exclusive_scan_i32(x)
    wd = dev(want)
    out = torch.empty_like(xd)
    for rep in range(3):
        _, tot = ssc.exclusive_scan(xd, out=out, scratch=scratch)
        assert torch.equal(out, wd) and int(host(tot)[0]) == total, rep
    inc = oracle.inclusive_scan_i32(x)
    ssc.inclusive_scan(xd, out=out, scratch=scratch)
    assert checks.first_mismatch(host(out), inc) == -1
    del out, wd
    f = wl.unit_float32(0x5CA8 + tiles, n)
    ref, ref_total = oracle.exclusive_scan_f32(f)
    fo, ftot = ssc.exclusive_scan(dev(f), scratch=scratch)
    max_rel, _, ok = checks.f32_scan_rel_errors(host(fo), ref)
    assert ok, max_rel
    assert abs(float(host(ftot)[0]) - ref_total) <= checks.F32_SCAN_REL_TOL * ref_total
    assert not ssc.timed_out(scratch)


def test_flag_selection_claim_paths_under_perturbation(perturbed):
    """Selection by flag bytes at 800 of its 61,440-flag tiles: the second and
    third tiles come from one claim (768 tiles or more on 256 compute units)."""
    n = 800 * 61440 + 5
    f = wl.flag_bytes(0x7AC5, n, 37)
    fw, mf = oracle.select_flags(f)
    fd = dev(f)
    scratch = ssc.new_scratch(n, fd.device)
    for rep in range(2):
        fidx, fcnt = ssc.select_flags(fd, scratch=scratch)
        assert int(host(fcnt)[0]) == mf and checks.first_mismatch(host(fidx)[:mf], fw) == -1, rep
    assert not ssc.timed_out(scratch)


def test_radix_sort_under_perturbation(perturbed):
    keys = wl.full_uint32(0x5EED7, 1 << 20)
    got = ssc.radix_sort4(dev(keys.view(np.int32)))
    assert checks.first_mismatch(host(got).view(np.uint32), oracle.radix_sort_u32(keys)) == -1
