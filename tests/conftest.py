import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running")


@pytest.fixture
def no_table():
    """Plans from the library's own rules only (the tuned table cleared for
    the test, the shipped table given back afterwards)."""
    import block_scaled_fp4_04_amd as nv
    nv.lib()
    nv.clear_plan_table()
    yield
    nv.load_default_plan_table()
