import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (HIP device) to run")
    config.addinivalue_line("markers", "slow: long-running (full-size shapes)")


def pytest_collection_modifyitems(config, items):
    # run GPU parity tests in a stable, cheap-first order; the fixed-scratch
    # forward's test file (test_zz_*) runs last of all
    def rank(it):
        if os.path.basename(str(it.fspath)).startswith("test_zz_"):
            return 2
        return 1 if it.get_closest_marker("slow") else 0

    items.sort(key=rank)
