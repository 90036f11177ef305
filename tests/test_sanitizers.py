"""CPU builds of the host planner and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer.

The planner (reduction_primitives_amd/csrc/rk_plan.cpp) does every call's
64-bit shape, stride, split and workspace arithmetic (AcceleratedKernels.jl
PR #176, "This PR"); tests/sanitize/plan_fuzz.cpp feeds it random layouts up
to the 2^62 limit and checks each plan's consistency, with any overflow or
out-of-bounds access fatal.  The oracle (oracle/oracle.c) is rebuilt the same
way and its pins (tests/test_oracle.py) run against that build.  Neither
needs a GPU; both use gcc's sanitizer runtimes.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "reduction_primitives_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-O1", "-g"]


def _have(tool):
    return shutil.which(tool) is not None


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(not _have("g++"), reason="needs g++")
def test_planner_fuzz_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "plan_fuzz")
    build = ["g++", "-std=c++17", *SAN, "-I" + CSRC, "-I" + os.path.join(ROOT, "include"),
             os.path.join(ROOT, "tests", "sanitize", "plan_fuzz.cpp"), os.path.join(CSRC, "rk_plan.cpp"), "-o", exe]
    proc = subprocess.run(build, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-3000:]
    for seed in (1, 2, 3):
        run = subprocess.run([exe, "300000", str(seed)], capture_output=True, text=True, timeout=300)
        assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
        assert run.stdout.startswith("ok "), run.stdout
        cases, accepted = int(run.stdout.split()[1]), int(run.stdout.split()[3])
        assert cases == 900000 and 0.2 * cases < accepted < cases    # both accepted and rejected layouts


@pytest.mark.skipif(not _have("gcc") or _asan_runtime() is None, reason="needs gcc with libasan")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    build = ["gcc", *SAN, "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared", "-o", lib,
             os.path.join(ROOT, "oracle", "oracle.c"), "-lm"]
    proc = subprocess.run(build, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-3000:]
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms       # the build is instrumented
    env = dict(os.environ, RKO_LIB=lib, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0")
    run = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"), "-q", "-x",
                          "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=600)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert " passed" in run.stdout and "ERROR: AddressSanitizer" not in run.stderr
