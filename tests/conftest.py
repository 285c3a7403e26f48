import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _library_built():
    """Build libevoattn.so once if it is not there yet (hipcc cross-compiles
    without a GPU); an existing build is used as is."""
    from evoformer_attention_amd import build, ops
    if not os.path.exists(ops.LIB_PATH):
        build.build()
    yield
