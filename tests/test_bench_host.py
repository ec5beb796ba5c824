"""Host-side parts of bench.py: the refusal of runs it does not measure, the
algorithmic byte and op counts behind its rates, and the roofline traffic figure's
tie to the kernel source it was measured on.  No GPU is used."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import moe_workloads as mw  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_step_counts_are_checked():
    for args in (("--steps", "0"), ("--warmup", "-1")):
        r = _run(*args)
        assert r.returncode == 2 and "--steps must be at least 1" in r.stderr


def test_without_a_gpu_it_exits_with_a_message():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu-baseline")
    assert r.returncode == 2 and "needs a GPU" in r.stderr and r.stdout == ""


def test_config_only_choices_cover_every_other_workload_line():
    r = _run("--help")
    assert r.returncode == 0
    for name in ("layer12288_uniform", "eplb4096", "decode96", "twohop46080", "batch_overlap"):
        assert name in r.stdout


def test_algorithmic_counts_of_the_12288_token_layer():
    """The per-step bytes and ops of T = 12288, H = 7168, k = 8, I = 2048, written
    out from the sizes: x read once as bf16 (176.2 MB), 98,304 messages of H + 16
    bytes (706.2 MB), the physical ids read and three row-index arrays written
    (4 bytes per route each, 1.6 MB), 16 bytes of metadata per (d, s); the combine
    reads 98,304 bf16 rows (1409.3 MB) and writes the bf16 output (176.2 MB); each
    route costs
    2·H·2I + 2·I·H = 88.08 M ops."""
    w = mw.WORKLOADS["layer12288"]
    assert (w.T, w.H, w.k, w.I, w.E, w.D, w.S) == (12288, 7168, 8, 2048, 256, 128, 128)
    a = bench.algorithmic(w)
    routes = 98304
    assert a["dispatch_bytes"] == 176_160_768 + routes * 7184 + routes * 4 * 4 + 128 * 128 * 16
    assert abs(a["dispatch_bytes"] / 1e6 - 884.2) < 0.1
    assert a["combine_bytes"] == routes * 14336 + routes * 8 + 176_160_768
    assert abs(a["combine_bytes"] / 1e6 - 1586.2) < 0.1
    assert a["dispatch_bytes"] + a["combine_bytes"] == 2_470_445_056
    assert a["gateup_ops"] == routes * 2 * 7168 * 4096
    assert a["down_ops"] * 2 == a["gateup_ops"]
    assert abs((a["gateup_ops"] + a["down_ops"]) / routes / 1e6 - 88.08) < 0.01
    assert abs((a["gateup_ops"] + a["down_ops"]) / 1e12 - 8.66) < 0.01
    # one scale per 256 columns: 28 per row at H = 7168
    assert a["combine_q8_bytes"] == routes * (7168 + 4 * 28) + routes * 8 + 176_160_768
    assert a["route_bytes"] == 12288 * 256 * 2 + routes * 12


def test_roofline_traffic_is_withheld_for_another_kernel_source(monkeypatch, tmp_path):
    """The committed counter figure is reported only for the source it was taken
    on: a changed GEMM source gives None."""
    assert bench.measured_traffic() is None or bench.measured_traffic() > 0
    other = tmp_path / "ffn_q8.hip"
    other.write_bytes(open(bench.GEMM_SRC, "rb").read() + b"\n// changed\n")
    monkeypatch.setattr(bench, "GEMM_SRC", str(other))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic() is None
