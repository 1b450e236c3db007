import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running on the CPU")


def pytest_collection_modifyitems(config, items):
    # GPU tests that run without a GPU fail loudly instead of passing on a fallback;
    # mark selection (-m "not gpu") keeps them out of CPU runs.
    pass
