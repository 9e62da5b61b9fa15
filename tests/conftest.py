import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: larger CPU case")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.build(force=not os.path.exists(os.path.join(ROOT, "oracle", "libq4ref.so")))
    return oracle


@pytest.fixture(autouse=True)
def _small_results_rel_l2():
    """Applies the relative L2 bar to the pooled small results of a GPU parity test."""
    mod = sys.modules.get("q4_gpu")
    if mod is not None:
        mod.SMALL.clear()
    yield
    mod = sys.modules.get("q4_gpu")
    if mod is not None:
        mod.check_small_pool()
