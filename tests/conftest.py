import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def oracle_lib():
    """The oracle; DS_SEL_TEST_ORACLE names another build of it (the sanitizer
    run), which then also serves every default oracle call."""
    import oracle
    path = os.environ.get("DS_SEL_TEST_ORACLE")
    if path:
        oracle._lib = oracle.load(path)
    return oracle.load()
