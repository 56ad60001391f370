import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """Compile the C oracle once per session if it is not there (gcc, a second or so)."""
    from oracle import oracle as orc
    if not os.path.exists(orc._LIB_PATH):
        orc.build_library(force=False)
    yield


@pytest.fixture(scope="session", autouse=True)
def _library_built():
    """Compile the HIP library in-tree if it is not there (hipcc cross-compiles on CPU)."""
    from hierarchical_kv_approximation_amd import lod
    if not os.path.exists(lod.LIB_PATH):
        from hierarchical_kv_approximation_amd import _build
        _build.build()
    yield
