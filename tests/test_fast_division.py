"""The INT8-return epilogue of the down projection replaces the per-element
division y / s by one reciprocal per row and a Markstein correction step.  That
is only sound if every INT8 code comes out the same as with the IEEE quotient:
checked here over every pair of bf16 values (y, amax), |y| <= amax, in C with
the same operation sequence (about 1.07e9 pairs)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_division_free_quotient_gives_the_ieee_codes(tmp_path):
    exe = str(tmp_path / "fastdiv")
    flags = ["-O2", "-ffp-contract=off", "-fopenmp"]
    # hardware FMA when the host has it (the same correctly rounded operation as libm's fmaf)
    probe = subprocess.run(["gcc", "-mfma", "-E", "-x", "c", "/dev/null"], capture_output=True)
    if probe.returncode == 0 and "fma" in open("/proc/cpuinfo").read():
        flags.append("-mfma")
    subprocess.run(["gcc", *flags, "-o", exe, os.path.join(HERE, "fastdiv_exhaustive.c"), "-lm"],
                   check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                         env={**os.environ, "OMP_NUM_THREADS": str(min(8, os.cpu_count() or 1))})
    print(res.stdout)
    assert res.returncode == 0, res.stdout
    pairs, fast, bad = (int(v) for v in res.stdout.split()[1::2])
    assert pairs == 1065402238 and bad == 0
    assert fast > 0.98 * pairs  # the division fallback is the rare tiny-scale case
