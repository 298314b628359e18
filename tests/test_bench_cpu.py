"""CPU checks of bench.py's contract: the one-GPU rule, the code-only kernel
source hash, and the traffic figure read from the committed rocprofv3 PMC
summary (a number only while that summary matches the kernel source)."""
from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
N_HEADLINE = 1 << 28


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a refused run


def test_kernel_hash_follows_code_not_comments():
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    assert bench._code_only(code) == bench._code_only("/* a note */ int f(int x) { return x + 1; }")
    assert bench._code_only(code) != bench._code_only(code.replace("x + 1", "x + 2"))
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0


def test_traffic_comes_from_a_matching_summary_only():
    with open(bench.PMC_SUMMARY) as f:
        text = f.read()
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip()
    for key in ("kernel_source_sha256_16", "hbm_bytes_per_launch", "fetch_bytes_per_launch",
                "write_bytes_per_launch", "algorithmic_bytes_per_launch"):
        assert key in fields, key
    got = bench.measured_traffic()
    if fields["kernel_source_sha256_16"] == bench.kernel_source_hash():
        # counted bytes of the headline launch: the input once, the survivors once
        alg = int(fields["algorithmic_bytes_per_launch"])
        assert got == int(float(fields["hbm_bytes_per_launch"]))
        assert alg == 4 * N_HEADLINE + 4 * 134_215_350
        assert alg <= got <= 1.02 * alg
        parts = int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
        assert abs(got - parts) <= 2  # the two passes' rounded shares
    else:
        assert got is None  # a summary of other code is never reported
