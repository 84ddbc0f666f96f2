import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU case")


@pytest.fixture(scope="session")
def lib():
    """The built C-ABI library (ctypes); builds it first if nothing is built."""
    import precision_moe_gemm_amd as pmg
    if not os.path.exists(pmg.library_path()):
        from precision_moe_gemm_amd import build
        build.build_library()
    return pmg.load_library()
