"""The allocation-free compaction entry point (ssc_compact_i32_noalloc)
against the entry point with a caller's scratch (ssc_compact_i32), through
the C ABI on the GPU: two calls in a row on the library's one scratch array,
the second on a smaller input, each equal to the existing entry point's
results bit for bit (count, survivors, ranks) with the rest of the output
untouched. The existing entry point is itself held to the oracle by the
parity suite."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import scan_stream_compaction_amd as ssc
from scan_stream_compaction_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _noalloc(x, pred, pa, pb, out, count, ranks):
    L = ssc.lib()
    rc = L.ssc_compact_i32_noalloc(x.data_ptr(), out.data_ptr(), x.numel(), pred, pa, pb,
                                   count.data_ptr(), None if ranks is None else ranks.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    assert rc == 0, ssc.lib().ssc_status_str(rc)


@pytest.mark.parametrize("cases", [
    # (seed, n, predicate, pa, pb, with ranks): two calls in a row, the second smaller
    ((0x5EED0B01, 3 * 30720 + 1234, ssc.PRED["mod_lt"], 10, 3, True),
     (0x5EED0B02, 30720 + 17, ssc.PRED["odd"], 0, 0, False)),
    ((0x5EED0B03, 2 ** 24 + 5, ssc.PRED["odd"], 0, 0, False),
     (0x5EED0B04, 65533, ssc.PRED["nonzero"], 0, 0, True)),
])
def test_noalloc_matches_the_entry_point_with_scratch(cases):
    for seed, n, pred, pa, pb, with_ranks in cases:
        x_np = wl.full_int32(seed, n)
        if pred == ssc.PRED["nonzero"]:
            x_np = wl.uniform_below(seed, n, 4)
        x = torch.from_numpy(x_np).to(DEV)
        ref_out, ref_cnt, ref_rk = ssc.compact(x, pred, pa, pb, ranks=True)
        out = torch.full_like(x, -7)
        cnt = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        rk = torch.full_like(x, -9) if with_ranks else None
        _noalloc(x, pred, pa, pb, out, cnt, rk)
        torch.cuda.synchronize()
        k = int(ref_cnt.item())
        assert int(cnt.item()) == k
        assert torch.equal(out[:k], ref_out[:k])
        assert bool((out[k:] == -7).all())
        if with_ranks:
            assert torch.equal(rk, ref_rk)
        want = x_np[(np.asarray(x_np) & 1).astype(bool)] if pred == ssc.PRED["odd"] else None
        if want is not None:
            assert np.array_equal(out[:k].cpu().numpy(), want)


def test_noalloc_binding_and_repeats():
    x = torch.from_numpy(wl.full_int32(0x5EED0B05, 100_000)).to(DEV)
    ref, rc = ssc.compact(x, "even")
    out = torch.empty_like(x)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    for _ in range(5):
        ssc.compact_noalloc(x, "even", out=out, count=cnt)
    torch.cuda.synchronize()
    k = int(rc.item())
    assert int(cnt.item()) == k and torch.equal(out[:k], ref[:k])
