"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This module holds only input generation: no predicate, scan, compaction or
partition arithmetic. Both the HIP path and the oracle receive the arrays it
returns, so they always see the same bytes.

Generator: the splitmix64 output function (Steele, Lea and Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014; Vigna's public-domain
splitmix64.c) evaluated on a counter, so any element can be produced
independently: ``z_i = mix64(seed + (i + 1) * 0x9E3779B97F4A7C15)``. Only the
high 32 bits ``h`` of ``z_i`` are used, except for 64-bit elements. Derived
values:

* uniform integer in ``[0, k)``: ``(h * k) >> 32``;
* full-range int32: ``h`` reinterpreted as two's complement;
* uniform fp32 in ``[0, 1)``: ``(h >> 8) * 2**-24`` (exact in fp32);
* full-range int64: all 64 bits of ``z_i``;
* flag bytes kept with probability p/100: ``0`` unless ``(h * 100) >> 32 < p``,
  else ``(h >> 24) | 1`` (any nonzero byte, odd so never 0).

The workloads follow the pages' own synthetic kinds: small uniform integers
with zeros to remove ("Day 33 compaction.cu"; "CIS 565 Project 2", whose
printed arrays hold values in [0, 4) and [0, 50)), the closed-form scan
inputs ``(i % 8) + 1`` ("Day 31 scan.cu") and "every fourth element 2.0f"
("Day 32 scan_2.cu"), full-range keys for the radix sort, and sizes that are
not multiples of a tile (8 Mi - 611, 2^16 - 3, 10^7).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix_hi32(seed: int, start: int, count: int) -> np.ndarray:
    """High 32 bits of splitmix64 outputs start .. start+count-1 (uint32)."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * GOLDEN_GAMMA
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
        return (z >> np.uint64(32)).astype(np.uint32)


def splitmix64(seed: int, n: int) -> np.ndarray:
    """Full 64-bit splitmix64 outputs 0..n-1 (small n; used by the pins)."""
    with np.errstate(over="ignore"):
        i = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * GOLDEN_GAMMA
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
        return z


def _mix64(seed: int, start: int, count: int) -> np.ndarray:
    """splitmix64 outputs start .. start+count-1 (uint64)."""
    with np.errstate(over="ignore"):
        i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * GOLDEN_GAMMA
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
        return z


def full_int64(seed: int, n: int, threads: int | None = None) -> np.ndarray:
    """int64 values over the whole range: all 64 bits of each output."""
    out = np.empty(n, np.uint64)
    starts = range(0, n, _CHUNK)

    def work(s):
        c = min(_CHUNK, n - s)
        out[s:s + c] = _mix64(seed, s, c)

    workers = threads or min(8, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(work, starts))
    return out.view(np.int64)


def hi32(seed: int, n: int, threads: int | None = None) -> np.ndarray:
    """High 32 bits of the first n splitmix64 outputs for `seed`, as uint32."""
    out = np.empty(n, np.uint32)
    if n <= _CHUNK:
        out[:] = _mix_hi32(seed, 0, n)
        return out
    starts = range(0, n, _CHUNK)

    def work(s):
        c = min(_CHUNK, n - s)
        out[s:s + c] = _mix_hi32(seed, s, c)

    workers = threads or min(8, os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(work, starts))
    return out


def uniform_below(seed: int, n: int, k: int) -> np.ndarray:
    """int32 values uniform in [0, k): (h * k) >> 32."""
    h = hi32(seed, n).astype(np.uint64)
    return ((h * np.uint64(k)) >> np.uint64(32)).astype(np.int32)


def full_int32(seed: int, n: int) -> np.ndarray:
    """int32 values over the whole range: h reinterpreted."""
    return hi32(seed, n).view(np.int32)


def full_uint32(seed: int, n: int) -> np.ndarray:
    return hi32(seed, n)


def unit_float32(seed: int, n: int) -> np.ndarray:
    """fp32 values uniform in [0, 1): (h >> 8) * 2^-24, exactly representable."""
    h = hi32(seed, n)
    return ((h >> np.uint32(8)).astype(np.float32) * np.float32(2.0 ** -24)).astype(np.float32)


def flag_bytes(seed: int, n: int, keep_pct: int) -> np.ndarray:
    """uint8 flags, nonzero with probability keep_pct / 100 (values 1..255)."""
    h = hi32(seed, n)
    keep = ((h.astype(np.uint64) * np.uint64(100)) >> np.uint64(32)) < np.uint64(keep_pct)
    return np.where(keep, (h >> np.uint32(24)) | np.uint32(1), np.uint32(0)).astype(np.uint8)


def mod8_plus1(n: int) -> np.ndarray:
    """int32 (i % 8) + 1."""
    return (np.arange(n, dtype=np.int64) % 8 + 1).astype(np.int32)


def every_fourth_two(n: int) -> np.ndarray:
    """fp32: 2.0 where i % 4 == 0, else 1.0."""
    x = np.ones(n, np.float32)
    x[0::4] = 2.0
    return x


# The five workloads (sizes, seeds, value recipes).
SEEDS = {1: 0x5EED0001, 2: 0x5EED0002, 3: 0x5EED0003, 4: 0x5EED0004, 5: 0x5EED0005}
N_SMALL_COMPACT = 65_533           # 2^16 - 3, values in [0, 4), nonzero kept
N_ZERO_REMOVAL = 8 * 1024 * 1024 - 611   # 8,387,997, values in [0, 10)
N_SCAN = 10_000_000
N_HEADLINE = 1 << 28               # full-range int32, odd kept
N_RADIX = 1 << 24                  # full-range uint32 keys
SWEEP_MOD = 100
SWEEP_KEEP = (1, 50, 99)


def small_compact_input() -> np.ndarray:
    return uniform_below(SEEDS[1], N_SMALL_COMPACT, 4)


def zero_removal_input() -> np.ndarray:
    return uniform_below(SEEDS[2], N_ZERO_REMOVAL, 10)


def scan_f32_input(n: int = N_SCAN) -> np.ndarray:
    return unit_float32(SEEDS[3], n)


def headline_input(n: int = N_HEADLINE) -> np.ndarray:
    return full_int32(SEEDS[4], n)


def radix_input(n: int = N_RADIX) -> np.ndarray:
    return full_uint32(SEEDS[5], n)
