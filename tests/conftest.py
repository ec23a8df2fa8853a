import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C-ABI library)")
    config.addinivalue_line("markers", "slow: full-size case, minutes of host work")


def pytest_collection_finish(session):
    # start the oracle's packing pool before any test touches the GPU
    if any(item.get_closest_marker("gpu") for item in session.items):
        from tests import oracle_cache
        oracle_cache.start_pool()


def pytest_sessionfinish(session, exitstatus):
    try:
        from tests import oracle_cache
        oracle_cache.stop_pool()
    except Exception:
        pass
