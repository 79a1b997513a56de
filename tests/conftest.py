import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _built_library():
    """Tests load the in-tree library; build it once only if nothing is built yet."""
    from mla_tree_verify_absorb_amd import _lib
    if not os.path.exists(_lib.library_path()):
        from mla_tree_verify_absorb_amd.build import build
        build()
    yield
