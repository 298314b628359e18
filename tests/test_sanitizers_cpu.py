"""The C code the tests trust, built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, static runtimes, every report fatal):

- oracle/oracle.c driven by tests/oracle_sanitize.c: every function over
  edge sizes (0 .. 30721) and every predicate, each buffer allocated at
  exactly the size the function may touch;
- tests/residue_fp64.c quick: the MOD_LT residue method check itself.

Host code only; nothing here touches a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-O1", "-g", "-std=c99", "-Wall", "-Wextra", "-Werror", "-fno-omit-frame-pointer",
       "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-static-libasan",
       "-static-libubsan"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")


def _build_and_run(tmp_path, name, sources, args=()):
    exe = tmp_path / name
    subprocess.run(["gcc", *SAN, *sources, "-o", str(exe), "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([str(exe), *args], capture_output=True, text=True, timeout=600, env=env)


def test_oracle_under_asan_and_ubsan(tmp_path):
    res = _build_and_run(tmp_path, "oracle_sanitize",
                         [os.path.join(HERE, "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "oracle.c")])
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok "), res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr


def test_residue_checker_under_asan_and_ubsan(tmp_path):
    res = _build_and_run(tmp_path, "residue_fp64", [os.path.join(HERE, "residue_fp64.c")], ["quick"])
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip() == "0 mismatches"
    assert "runtime error" not in res.stderr, res.stderr
