"""CPU code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two host programs are built here with -fsanitize=address,undefined (every finding fatal) and
run: tests/host/plan_bounds.cpp, the bounds harness of the library's plans and workspace
carving (ss_plan.h: the workloads, shapes past 2^31 elements, a seeded sweep of the option
space, invalid and overflowing dims), and tests/host/oracle_driver.c, which drives the C fp64
oracle (oracle/ss_oracle.c) through its forward and backward on small shapes with OpenMP on
two threads.  The harness's self-test must report a planted overlap.  No GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2",
           UBSAN_OPTIONS="print_stacktrace=1")


def _build(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_bounds_sanitized(tmp_path):
    exe = str(tmp_path / "plan_bounds")
    _build(["g++", "-std=c++17", *SAN, f"-I{ROOT}/include",
            f"-I{ROOT}/selective_state_space_34_amd/csrc", "-I/opt/rocm/include",
            "-D__HIP_PLATFORM_AMD__", f"{ROOT}/tests/host/plan_bounds.cpp", "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("plan bounds ok"), r.stdout
    assert int(r.stdout.split()[-1]) > 40000
    planted = subprocess.run([exe, "selftest"], capture_output=True, text=True, timeout=60, env=ENV)
    assert planted.returncode == 1 and "FAIL overlap" in planted.stdout, planted.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_sanitized(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _build(["gcc", "-std=c11", *SAN, "-fopenmp", f"{ROOT}/oracle/ss_oracle.c",
            f"{ROOT}/tests/host/oracle_driver.c", "-lm", "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("oracle ok"), r.stdout
