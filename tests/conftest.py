import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X) and the built HIP library")
    config.addinivalue_line("markers", "slow: large inputs (seconds to minutes)")


def pytest_collection_modifyitems(config, items):
    # make sure the oracle is compiled once before any test imports it
    try:
        import oracle
        oracle.build()
    except Exception:  # pragma: no cover - reported by the tests themselves
        pass
