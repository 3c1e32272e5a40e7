import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    if not os.environ.get("PAGED_ORACLE_LIB"):  # a mutation run brings its own build
        import oracle
        oracle.build()
    yield
