import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running full-size case")


@pytest.fixture(scope="session")
def root_dir():
    return ROOT


def pytest_sessionstart(session):
    """Build the HIP library only if nothing is built yet."""
    from mixture_experts_ffn_rmsnorm_amd import build, moe

    if not os.path.exists(moe.LIB_PATH):
        build.build(verbose=False)
