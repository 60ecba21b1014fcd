import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running oracle case")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="session")
def ropelib():
    """The built librope_fa.so (built first if absent), loaded through the binding."""
    import rope_flashattention_amd as rfa
    if not os.path.exists(rfa.LIB_PATH):
        from rope_flashattention_amd.build import build
        build()
    return rfa.lib()
