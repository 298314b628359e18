"""The MOD_LT predicate's fp64 residue method (the fraction of
fma(x, 1/m, 1/(2m)) against s/m), checked on the host against 64-bit integer
residues (tests/residue_fp64.c): the ends and the middle of the int32 range
for small, prime and the largest moduli with bounds inside and outside
[1, m - 1], and 5e7 random (x, m, s) triples with s from -1 to m + 1.
`residue_fp64 full` sweeps all 2^32 x."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fp64_residue_method_matches_integer_residue(tmp_path):
    exe = tmp_path / "residue_fp64"
    subprocess.run(["gcc", "-O2", "-std=c99", "-Wall", "-Werror", os.path.join(HERE, "residue_fp64.c"),
                    "-o", str(exe), "-lm"], check=True)
    res = subprocess.run([str(exe), "quick"], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip() == "0 mismatches"
