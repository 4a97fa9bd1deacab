import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle work at DiT sizes (tens of seconds on the CPU)")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (never silently skip) when the device is missing;
    # select them with -m gpu on a GPU machine, -m "not gpu" elsewhere.
    pass
