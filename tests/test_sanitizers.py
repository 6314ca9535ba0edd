"""Sanitizer tier (CPU only): the host code that takes no GPU, built with
g++/gcc under AddressSanitizer and UndefinedBehaviorSanitizer, every finding
fatal.

* The planning code the library runs before any launch (argument checks,
  variant choice, grid, the workgroup -> tile map): tests/sanitize/plan_check.cpp
  drives it over an argument table and a sweep, and checks the tile map is a
  bijection.
* The oracle (oracle/tgemm_ref.c): a sanitized build of it runs the oracle's
  pin tests (test_oracle.py, test_oracle_ex.py) in a child process with the
  sanitizer runtime preloaded.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="no host compiler")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_planning_code_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "dense_tiled_gemm_tgemm_amd", "csrc"),
           os.path.join(ROOT, "tests", "sanitize", "plan_check.cpp"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "all expectations held" in run.stdout


def test_oracle_pins_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no libasan runtime")
    from oracle import build as oracle_build
    lib = oracle_build.build(sanitize=True, out=str(tmp_path / "liboracle_tgemm_san.so"))
    env = dict(os.environ, TGEMM_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle.py"),
                          os.path.join(ROOT, "tests", "test_oracle_ex.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out
    assert " passed" in out
