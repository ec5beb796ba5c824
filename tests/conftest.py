"""Shared pytest setup: the `gpu` marker, build-on-demand, and common fixtures."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes on the CPU side)")


def _ensure_built():
    import __graft_entry__ as ge
    need = [os.path.join(ROOT, "oracle", "libmoe_oracle.so"),
            os.path.join(ROOT, "combine_moe_route_topk_amd", "libmoe_route_topk.so")]
    if not all(os.path.exists(p) for p in need):
        ge.build()


_ensure_built()


@pytest.fixture(scope="session")
def gpu_available():
    import torch
    return torch.cuda.is_available()
