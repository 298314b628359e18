"""Host-side checks of the C ABI, runnable without a GPU.

The library must load and export every function include/ssc.h declares, the
enum numbering must agree with the oracle's and the binding's, and every
argument error must be reported before the library touches HIP. The pointer
values used here are never dereferenced: each call is rejected by the argument
checks that run before anything is enqueued.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import oracle
import scan_stream_compaction_amd as ssc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssc.h")

OK, ARG, SIZE, ALIAS, SCRATCH, HIP, DEVICE = range(7)
INT32_MAX = 2**31 - 1

# Fake, never-dereferenced device addresses, 256-byte aligned and far apart.
A = 0x7F0000000000
B = 0x7F1000000000
C = 0x7F2000000000
S = 0x7F3000000000


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(ssc_[a-z0-9_]+)\s*\(", text))


def _enum(name):
    text = open(HEADER).read()
    body = re.search(r"typedef enum %s \{(.*?)\}" % name, text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    return {k: int(v) for k, v in re.findall(r"(\w+)\s*=\s*(\d+)", body)}


def test_library_exports_every_declared_symbol():
    L = ssc.lib()
    declared = _declared()
    assert declared == set(ssc.SIGNATURES), declared ^ set(ssc.SIGNATURES)
    for name in declared:
        assert hasattr(L, name), name


@pytest.mark.parametrize("path", [ssc.PERTURB_LIB_PATH, ssc.STRESS_LIB_PATH])
def test_test_builds_export_every_symbol_and_size_their_scratch(path):
    """The race tests' builds: the same C ABI; the stress build's tiles are
    3840 elements, so its scratch holds 16 bytes of descriptors per 3840
    elements and it refuses n beyond 2^17 of its tiles."""
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} not built (python -m scan_stream_compaction_amd.build)")
    L = ssc.load_library(path)
    for name in _declared():
        assert hasattr(L, name), name
    stress = path == ssc.STRESS_LIB_PATH
    T = L.ssc_tile_elems()
    assert T == (3840 if stress else 30720)
    for n in (1, T, T + 1, 2**28):
        assert L.ssc_scratch_bytes(n) == 512 + 16 * ((n + T - 1) // T)
    big = (1 << 17) * 3840 + 1
    rc = L.ssc_compact_i32(None, None, big, 1, 0, 0, None, None, None, 0, None)
    code = {v: k for k, v in ssc.STATUS.items()}
    assert rc == (code["SSC_ERR_SIZE"] if stress else code["SSC_ERR_ARG"])


def test_enum_numbering_agrees_with_oracle_and_binding():
    preds = _enum("ssc_pred")
    assert preds == {"SSC_PRED_NONZERO": 0, "SSC_PRED_ODD": 1, "SSC_PRED_EVEN": 2,
                     "SSC_PRED_BIT_SET": 3, "SSC_PRED_BIT_CLEAR": 4, "SSC_PRED_MOD_LT": 5,
                     "SSC_PRED_F32_NONZERO": 6, "SSC_PRED_F32_GT": 7, "SSC_PRED_F32_LT": 8,
                     "SSC_PRED_F32_IN": 9}
    for k, v in preds.items():
        assert ssc.PRED[k[len("SSC_PRED_"):].lower()] == v
        assert oracle.lib().orc_pred_id(v) == v
    assert (oracle.PRED_NONZERO, oracle.PRED_ODD, oracle.PRED_EVEN, oracle.PRED_BIT_SET,
            oracle.PRED_BIT_CLEAR, oracle.PRED_MOD_LT) == tuple(range(6))
    assert (oracle.PRED_F32_NONZERO, oracle.PRED_F32_GT, oracle.PRED_F32_LT,
            oracle.PRED_F32_IN) == tuple(range(6, 10))
    st = _enum("ssc_status")
    assert {v: k for k, v in st.items()} == ssc.STATUS


def test_tile_and_scratch_sizes():
    L = ssc.lib()
    T = L.ssc_tile_elems()
    assert T == 30720          # 15 data wavefronts x 2048 elements (2 rounds of 1024 in a scan)
    # a 512-byte header, then two 8-byte descriptor words per tile (the fp32
    # scans' descriptors are two words wide)
    for n in (0, 1, T - 1, T, T + 1, 2**28, INT32_MAX):
        tiles = (n + T - 1) // T
        assert L.ssc_scratch_bytes(n) == 512 + 16 * tiles
        assert L.ssc_radix_sort_scratch_bytes(n) == 512 + 16 * tiles
    assert L.ssc_scratch_bytes(INT32_MAX) == 512 + 16 * 69906
    assert L.ssc_scratch_bytes(-5) == 512
    # 4-bit radix sort: a scan scratch (256-byte rounded) for the 16 x tiles
    # count table, then the table
    for n in (1, 8191, 8192, 8193, 2**24, INT32_MAX):
        rt = (n + 8191) // 8192
        scan = 512 + 16 * ((16 * rt + T - 1) // T)
        assert L.ssc_radix_sort4_scratch_bytes(n) == (scan + 255) // 256 * 256 + 64 * rt
    assert L.ssc_radix_sort4_scratch_bytes(0) == 512
    assert L.ssc_radix_sort4_scratch_bytes(INT32_MAX) == 2816 + 64 * 262144


def test_status_strings():
    L = ssc.lib()
    for s in range(7):
        assert L.ssc_status_str(s)
    assert L.ssc_status_str(99) == b"unknown status"
    assert L.ssc_last_hip_error() == 0


def _compact(**kw):
    a = dict(inp=A, out=B, n=1000, pred=1, pa=0, pb=0, count=C, ranks=None, scratch=S,
             sbytes=1 << 20, stream=None)
    a.update(kw)
    return ssc.lib().ssc_compact_i32(a["inp"], a["out"], a["n"], a["pred"], a["pa"], a["pb"],
                                     a["count"], a["ranks"], a["scratch"], a["sbytes"],
                                     a["stream"])


def test_compact_argument_errors():
    assert _compact(inp=None) == ARG
    assert _compact(out=None) == ARG
    assert _compact(count=None) == ARG
    assert _compact(n=-1) == ARG
    assert _compact(n=INT32_MAX + 1) == SIZE
    assert _compact(pred=6) == ARG
    assert _compact(pred=-1) == ARG
    assert _compact(pred=3, pa=32) == ARG
    assert _compact(pred=4, pa=-1) == ARG
    assert _compact(pred=5, pa=0) == ARG
    assert _compact(inp=A + 2) == ARG          # not 4-byte aligned
    assert _compact(count=C + 1) == ARG
    assert _compact(out=A + 400) == ALIAS      # out overlaps in
    assert _compact(count=A + 4) == ALIAS
    assert _compact(ranks=B + 8) == ALIAS
    assert _compact(scratch=None) == SCRATCH
    assert _compact(scratch=S + 4) == SCRATCH  # not 8-byte aligned
    assert _compact(sbytes=511) == SCRATCH
    assert _compact(n=40000, sbytes=512 + 16) == SCRATCH  # needs two tiles' descriptors
    assert _compact(scratch=A) == ALIAS


def test_scan_partition_atomic_sort_copy_argument_errors():
    L = ssc.lib()
    big = 1 << 20
    # scan: exact in-place is legal (checked later on the GPU); partial overlap is not
    assert L.ssc_exclusive_scan_i32(A, A + 4, 100, None, S, big, None) == ALIAS
    assert L.ssc_exclusive_scan_f32(A, B, 100, A + 8, S, big, None) == ALIAS
    assert L.ssc_exclusive_scan_i32(None, B, 100, None, S, big, None) == ARG
    assert L.ssc_exclusive_scan_i32(A, B, -3, None, S, big, None) == ARG
    assert L.ssc_exclusive_scan_i32(A, B, INT32_MAX + 1, None, S, big, None) == SIZE
    assert L.ssc_exclusive_scan_f32(A, B, 100, None, S, 100, None) == SCRATCH
    assert L.ssc_exclusive_scan_f32(A, B + 2, 100, None, S, big, None) == ARG
    # partition: in-place is not allowed
    assert L.ssc_partition_i32(A, A, 100, 2, 0, 0, C, S, big, None) == ALIAS
    assert L.ssc_partition_i32(A, B, 100, 9, 0, 0, C, S, big, None) == ARG
    assert L.ssc_partition_i32(A, B, 100, 2, 0, 0, None, S, big, None) == ARG
    assert L.ssc_partition_i32(A, B, 100, 2, 0, 0, C, S, 8, None) == SCRATCH
    # count_if
    assert L.ssc_count_if_i32(A, 100, 0, 0, 0, A + 8, S, big, None) == ALIAS
    assert L.ssc_count_if_i32(A, 100, 5, 0, 0, C, S, big, None) == ARG
    assert L.ssc_count_if_i32(A, 100, 0, 0, 0, C, S, 100, None) == SCRATCH
    assert L.ssc_count_if_i32(A, 100, 0, 0, 0, C, A, big, None) == ALIAS
    # scratch_init rejects what it cannot clear, before touching HIP
    assert L.ssc_scratch_init(None, big, None) == SCRATCH
    assert L.ssc_scratch_init(S + 4, big, None) == SCRATCH
    assert L.ssc_scratch_init(S, 100, None) == SCRATCH
    # atomic
    assert L.ssc_compact_atomic_i32(A, B, 100, 1, 0, 0, C, 2, None) == ARG
    assert L.ssc_compact_atomic_i32(A, A + 8, 100, 1, 0, 0, C, 0, None) == ALIAS
    # radix sort: tmp must not overlap; scratch must hold 32 descriptor arrays
    assert L.ssc_radix_sort_u32(A, B, B + 64, 100, S, big, None) == ALIAS
    assert L.ssc_radix_sort_u32(A, B, C, 100, S, 512 + 7, None) == SCRATCH
    assert L.ssc_radix_sort_u32(A, B, None, 100, S, big, None) == ARG
    # 4-bit radix sort: passes 1..8; out == in only with an even pass count
    assert L.ssc_radix_sort4_u32(A, B, C, 100, 0, S, big, None) == ARG
    assert L.ssc_radix_sort4_u32(A, B, C, 100, 9, S, big, None) == ARG
    assert L.ssc_radix_sort4_u32(A, A, C, 100, 3, S, big, None) == ALIAS
    assert L.ssc_radix_sort4_u32(A, B, B + 64, 100, 8, S, big, None) == ALIAS
    assert L.ssc_radix_sort4_u32(A, B, None, 100, 8, S, big, None) == ARG
    assert L.ssc_radix_sort4_u32(A, B, C, 100, 8, S, 512 + 7, None) == SCRATCH
    assert L.ssc_radix_sort4_u32(A, B, C, 100, 8, A, big, None) == ALIAS
    # inclusive scans: same rules as the exclusive ones
    assert L.ssc_inclusive_scan_i32(A, A + 4, 100, None, S, big, None) == ALIAS
    assert L.ssc_inclusive_scan_f32(A, B, 100, B + 8, S, big, None) == ALIAS
    assert L.ssc_inclusive_scan_i32(A, None, 100, None, S, big, None) == ARG
    assert L.ssc_inclusive_scan_i32(A, B, INT32_MAX + 1, None, S, big, None) == SIZE
    assert L.ssc_inclusive_scan_f32(A, B, 100, None, S, 100, None) == SCRATCH
    # selection: no overlap, predicate arguments checked, scratch sized
    assert L.ssc_select_index_i32(A, A + 8, 100, 1, 0, 0, C, S, big, None) == ALIAS
    assert L.ssc_select_index_i32(A, B, 100, 1, 0, 0, B + 4, S, big, None) == ALIAS
    assert L.ssc_select_index_i32(A, B, 100, 5, 0, 0, C, S, big, None) == ARG
    assert L.ssc_select_index_i32(A, B, 100, 1, 0, 0, None, S, big, None) == ARG
    assert L.ssc_select_index_i32(A, B, -1, 1, 0, 0, C, S, big, None) == ARG
    assert L.ssc_select_index_i32(A, B, 100, 1, 0, 0, C, S, 100, None) == SCRATCH
    assert L.ssc_select_index_i32(A, B, 100, 1, 0, 0, C, B, big, None) == ALIAS
    # fp32 calls take predicates 6..9 only, int32 calls 0..5 only
    for p in (0, 5, 10, -1):
        assert L.ssc_compact_f32(A, B, 100, p, 0.0, 0.0, C, None, S, big, None) == ARG
        assert L.ssc_partition_f32(A, B, 100, p, 0.0, 0.0, C, S, big, None) == ARG
        assert L.ssc_select_index_f32(A, B, 100, p, 0.0, 0.0, C, S, big, None) == ARG
    for p in (6, 9):
        assert L.ssc_compact_i32(A, B, 100, p, 0, 0, C, None, S, big, None) == ARG
        assert L.ssc_partition_i32(A, B, 100, p, 0, 0, C, S, big, None) == ARG
        assert L.ssc_count_if_i32(A, 100, p, 0, 0, C, S, big, None) == ARG
    assert L.ssc_compact_f32(A, A + 8, 100, 7, 0.5, 0.0, C, None, S, big, None) == ALIAS
    assert L.ssc_partition_f32(A, B, 100, 9, 0.0, 1.0, None, S, big, None) == ARG
    assert L.ssc_select_index_f32(A, B, 100, 6, 0.0, 0.0, C, S, 100, None) == SCRATCH
    # multi-launch comparison pipelines
    # levels of 8193, 2 and 1 tile sums, each rounded up to 4 words
    assert L.ssc_multipass_scratch_bytes(8192 * 8192 + 1) == 4 * (8196 + 4 + 4) + 256
    assert L.ssc_exclusive_scan_multipass_i32(A, A + 4, 100, None, S, big, None) == ALIAS
    assert L.ssc_exclusive_scan_multipass_i32(A, B, 100, None, S + 8, big, None) == SCRATCH
    assert L.ssc_exclusive_scan_multipass_i32(A, B, 100, None, S, 100, None) == SCRATCH
    assert L.ssc_compact_multipass_i32(A, B, 100, 1, 0, 0, C, None, S, big, None) == ARG
    assert L.ssc_compact_multipass_i32(A, B, 100, 1, 0, 0, C, B + 8, S, big, None) == ALIAS
    assert L.ssc_compact_multipass_i32(A, B, 100, 7, 0, 0, C, C + 64, S, big, None) == ARG
    # copy
    assert L.ssc_copy_i32(A, A + 4, 100, None) == ALIAS
    assert L.ssc_copy_i32(A, B, -1, None) == ARG
    # the multi-launch compaction's separate steps
    assert L.ssc_mark_i32(A, A + 8, 100, 1, 0, 0, None) == ALIAS
    assert L.ssc_mark_i32(A, B, 100, 4, 32, 0, None) == ARG
    assert L.ssc_mark_i32(None, B, 100, 1, 0, 0, None) == ARG
    assert L.ssc_mark_i32(A, B, INT32_MAX + 1, 1, 0, 0, None) == SIZE
    assert L.ssc_scatter_i32(A, B, C, 100, 1, 0, 0, None, None) == ARG
    assert L.ssc_scatter_i32(A, B, B + 8, 100, 1, 0, 0, C, None) == ALIAS
    assert L.ssc_scatter_i32(A, B, C, 100, 1, 0, 0, A + 12, None) == ALIAS
    assert L.ssc_scatter_i32(A, B, C, 100, 5, 0, 0, C + 4096, None) == ARG
    # the allocation-free compaction: the same argument checks, before any HIP call
    assert L.ssc_compact_i32_noalloc(A, B, 100, 1, 0, 0, None, None, None) == ARG
    assert L.ssc_compact_i32_noalloc(A, A + 8, 100, 1, 0, 0, C, None, None) == ALIAS
    assert L.ssc_compact_i32_noalloc(A, B, 100, 1, 0, 0, C, A + 40, None) == ALIAS
    assert L.ssc_compact_i32_noalloc(A, B, 100, 4, 32, 0, C, None, None) == ARG
    assert L.ssc_compact_i32_noalloc(A, B, 100, 6, 0, 0, C, None, None) == ARG
    assert L.ssc_compact_i32_noalloc(A, B, -1, 1, 0, 0, C, None, None) == ARG
    assert L.ssc_compact_i32_noalloc(A, B, INT32_MAX + 1, 1, 0, 0, C, None, None) == SIZE
    assert L.ssc_compact_i32_noalloc(A, B + 2, 100, 1, 0, 0, C, None, None) == ARG
    # the time-out check reads a scratch header into a device int outside it
    assert L.ssc_scratch_timed_out(None, big, C, None) == SCRATCH
    assert L.ssc_scratch_timed_out(S + 4, big, C, None) == SCRATCH
    assert L.ssc_scratch_timed_out(S, 100, C, None) == SCRATCH
    assert L.ssc_scratch_timed_out(S, big, None, None) == ARG
    assert L.ssc_scratch_timed_out(S, big, C + 2, None) == ARG
    assert L.ssc_scratch_timed_out(S, big, S + 8, None) == ALIAS


def test_flag_pair_and_64bit_argument_errors():
    L = ssc.lib()
    big = 1 << 20
    D = 0x7F4000000000
    # flag bytes: 4-byte aligned flags, no overlap, scratch sized
    assert L.ssc_compact_flags_b32(A, B + 2, C, 100, D, S, big, None) == ARG
    assert L.ssc_compact_flags_b32(None, B, C, 100, D, S, big, None) == ARG
    assert L.ssc_compact_flags_b32(A, B, C, 100, None, S, big, None) == ARG
    assert L.ssc_compact_flags_b32(A, A + 396, C, 100, D, S, big, None) == ALIAS  # flags inside in
    assert L.ssc_compact_flags_b32(A, B, B + 96, 100, D, S, big, None) == ALIAS   # out over flags
    assert L.ssc_compact_flags_b32(A, B, C, 100, D, S, 100, None) == SCRATCH
    assert L.ssc_compact_flags_b32(A, B, C, 100, D, B, big, None) == ALIAS
    assert L.ssc_compact_flags_b32(A, B, C, INT32_MAX + 1, D, S, big, None) == SIZE
    assert L.ssc_select_flags(B, C, 100, C + 8, S, big, None) == ALIAS
    assert L.ssc_select_flags(B + 1, C, 100, D, S, big, None) == ARG
    assert L.ssc_select_flags(None, C, 100, D, S, big, None) == ARG
    assert L.ssc_select_flags(B, C, -2, D, S, big, None) == ARG
    # key-value: every pair of the four arrays and the count apart
    assert L.ssc_compact_kv_i32(A, A + 200, C, D, 100, 1, 0, 0, S, S + 4096, big, None) == ALIAS
    assert L.ssc_compact_kv_i32(A, B, C, C + 8, 100, 1, 0, 0, S, S + 4096, big, None) == ALIAS
    assert L.ssc_compact_kv_i32(A, B, C, D, 100, 1, 0, 0, D + 12, S + 4096, big, None) == ALIAS
    assert L.ssc_compact_kv_i32(A, B, C, D, 100, 6, 0, 0, S, S + 4096, big, None) == ARG
    assert L.ssc_compact_kv_i32(A, B, C, D, 100, 3, 32, 0, S, S + 4096, big, None) == ARG
    assert L.ssc_compact_kv_i32(A, B + 2, C, D, 100, 1, 0, 0, S, S + 4096, big, None) == ARG
    assert L.ssc_compact_kv_i32(A, B, C, None, 100, 1, 0, 0, S, S + 4096, big, None) == ARG
    assert L.ssc_compact_kv_i32(A, B, C, D, 100, 1, 0, 0, S, S + 4096, 100, None) == SCRATCH
    for p in (0, 5, 10):
        assert L.ssc_compact_kv_f32(A, B, C, D, 100, p, 0.0, 0.0, S, S + 4096, big, None) == ARG
    # 64-bit elements: bits 0..63, no residue or fp32 predicates, 8-byte alignment
    assert L.ssc_compact_i64(A, B, 100, 3, 64, C, S, big, None) == ARG
    assert L.ssc_compact_i64(A, B, 100, 4, -1, C, S, big, None) == ARG
    assert L.ssc_compact_i64(A, B, 100, 5, 100, C, S, big, None) == ARG
    assert L.ssc_compact_i64(A, B, 100, 6, 0, C, S, big, None) == ARG
    assert L.ssc_compact_i64(A + 4, B, 100, 1, 0, C, S, big, None) == ARG
    assert L.ssc_compact_i64(A, B + 4, 100, 1, 0, C, S, big, None) == ARG
    assert L.ssc_compact_i64(A, A + 792, 100, 1, 0, C, S, big, None) == ALIAS  # in is 800 bytes
    assert L.ssc_compact_i64(A, B, 100, 1, 0, B + 796, S, big, None) == ALIAS
    assert L.ssc_compact_i64(A, B, 100, 1, 0, C, S, 100, None) == SCRATCH
    assert L.ssc_select_index_i64(A, A + 792, 100, 1, 0, C, S, big, None) == ALIAS
    assert L.ssc_select_index_i64(A, B, 100, 3, 63, None, S, big, None) == ARG
    assert L.ssc_select_index_i64(A, B, 100, 2, 0, C, A, big, None) == ALIAS


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(16, dtype=torch.int32)
    with pytest.raises(ValueError):
        ssc.compact(x, "odd")
    with pytest.raises(ValueError):
        ssc.exclusive_scan(x)
    with pytest.raises(ValueError):
        ssc.timed_out(torch.zeros(1024, dtype=torch.uint8))


def test_binding_argument_checker():
    """The checker every caller-supplied tensor goes through: it refuses what
    is not a tensor and what is not on the GPU before looking further (on the
    GPU the dtype, device and size checks follow; tested there)."""
    import torch
    x = torch.zeros(16, dtype=torch.int32)
    with pytest.raises(TypeError):
        ssc._need([0] * 16, "out", x, (torch.int32,), 16)
    with pytest.raises(ValueError, match="GPU"):
        ssc._need(torch.zeros(16, dtype=torch.int32), "out", x, (torch.int32,), 16)
