"""Build libssc.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m scan_stream_compaction_amd.build [--asm DIR]
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


def build(asm_dir: str | None = None) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *flags(), "-shared", SRC, "-o", tmp]
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        cmd += ["-save-temps=obj"]
        cwd = asm_dir
        cmd[-1] = os.path.abspath(tmp)
    else:
        cwd = ROOT
    subprocess.run(cmd, check=True, cwd=cwd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="keep intermediate files (ISA) in this directory")
    a = ap.parse_args()
    print(build(a.asm))
    sys.exit(0)
