import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads (seconds to minutes of host work)")


import pytest  # noqa: E402


@pytest.fixture(scope="session", autouse=True)
def _built_library():
    """Build libfgg.so in-tree if it is missing (never when it exists)."""
    from fp4_grouped_gemm_amd import library_path
    if not os.path.exists(library_path()):
        from fp4_grouped_gemm_amd.build import build
        build()
    yield
