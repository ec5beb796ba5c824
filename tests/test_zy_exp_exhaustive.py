"""The SwiGLU epilogue's exponential agrees with the oracle's for every input.

Both sides define e = fp32(exp(-(double)g)); the GPU evaluates exp with the
device math library, the oracle with the host C library.  h = (g / (1 + e)) * u
is then the same IEEE expression on both sides, so the gate/up outputs, and the
requantized hq, hs that feed the down projection, are bit-equal for any input
exactly when the two exponentials agree.  ``exp_exhaustive.hip`` (built by
``__graft_entry__.build()``) checks all 4,278,190,082 non-NaN fp32 inputs.
The file name sorts last so that a failure here never stops the parity tests
of a ``pytest -x`` run before they have run.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "exp_exhaustive")


@pytest.mark.gpu
def test_device_exp_equals_host_exp_for_every_fp32_input():
    assert os.path.exists(EXE), f"{EXE} is not built: run __graft_entry__.build()"
    print("[case] exp over all fp32 inputs", flush=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=300,
                         env={**os.environ, "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS", "16")})
    print(res.stdout[-2000:])
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    last = res.stdout.strip().splitlines()[-1].split()
    assert last[0] == "inputs" and int(last[1]) == 4278190082 and int(last[3]) == 0
