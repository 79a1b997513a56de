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
    """Tests load the in-tree library: build it if it is missing or was built from other sources (the
    library carries a digest of its sources; the binding refuses a mismatch)."""
    from mla_tree_verify_absorb_amd import _lib
    if not _lib.is_current():
        from mla_tree_verify_absorb_amd.build import build
        build()
    yield
