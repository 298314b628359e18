"""Build libssc.so (HIP, gfx950) in-tree with hipcc.

Also builds two test builds of the same sources for the race tests:
- libssc_perturb.so (-DSSC_PERTURB): every tile claim, descriptor
  publication, arrival and look-back poll pauses for a hashed number of
  clocks, so tiles finish in other orders;
- libssc_stress.so (-DSSC_STRESS_TILES): the persistent kernels' tiles are
  eight times smaller, so a call makes eight times the claims, descriptors
  and look-backs.
The library proper contains neither.

Usage: python -m scan_stream_compaction_amd.build [--asm DIR] [--only lib|perturb|stress]
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ssc.hip")
LIB = os.path.join(PKG, "libssc.so")
PERTURB_LIB = os.path.join(PKG, "libssc_perturb.so")
STRESS_LIB = os.path.join(PKG, "libssc_stress.so")

ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libssc.so)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # Packed fp32 instructions stay off: the compiler must not form them.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
    ]


def _command(out: str, defines: list[str], asm_dir: str | None) -> tuple[list[str], str]:
    cmd = [hipcc(), *flags(), *defines, "-shared", SRC, "-o", out]
    cwd = ROOT
    if asm_dir:
        # intermediate files (device ISA included) go next to the output
        os.makedirs(asm_dir, exist_ok=True)
        cmd += ["-save-temps=cwd"]
        cwd = asm_dir
    return cmd, cwd


def build(asm_dir: str | None = None, only: str | None = None) -> list[str]:
    """Compile the library and the two test builds (or only the one named)
    in parallel; each output is replaced only once it is complete."""
    jobs = []
    for name, out, defines in (("lib", LIB, []), ("perturb", PERTURB_LIB, ["-DSSC_PERTURB=1"]),
                               ("stress", STRESS_LIB, ["-DSSC_STRESS_TILES=1"])):
        if only and only != name:
            continue
        cmd, cwd = _command(out + ".tmp", defines, asm_dir if name == "lib" else None)
        jobs.append((out, subprocess.Popen(cmd, cwd=cwd)))
    failed = [out for out, p in jobs if p.wait() != 0]
    if failed:
        raise RuntimeError(f"hipcc failed for {', '.join(failed)}")
    for out, _ in jobs:
        os.replace(out + ".tmp", out)
    return [out for out, _ in jobs]


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="keep intermediate files (ISA) of libssc.so in this directory")
    ap.add_argument("--only", choices=("lib", "perturb", "stress"), default=None)
    a = ap.parse_args()
    print("\n".join(build(a.asm, a.only)))
    sys.exit(0)
