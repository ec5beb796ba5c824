"""The CPU side under AddressSanitizer and UndefinedBehaviorSanitizer: the oracle
(oracle/moe_oracle.c) and the library's host-only code (csrc/host.cpp: geometry
validation, static sizing, scratch layouts, the replica planner) are built with
gcc/g++ and both sanitizers (no GPU code is involved) and driven on tiny and
random inputs; any memory error, leak or undefined behaviour fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                    reason="needs gcc and g++")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-ffp-contract=off", "-fopenmp", *SAN, "-o", exe,
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"], ROOT)
    assert "oracle driver ok" in _run([exe], ROOT)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-o", exe,
          os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"),
          os.path.join(ROOT, "combine_moe_route_topk_amd", "csrc", "host.cpp")], ROOT)
    assert "host driver ok" in _run([exe], ROOT)
