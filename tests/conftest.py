import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _library_built():
    """Build libvpk.so in-tree only if nothing is built yet."""
    from varlen_paged_kv_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from varlen_paged_kv_amd import build
        build.build()
    yield
