import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run with -m gpu")
    config.addinivalue_line("markers", "slow: large CPU work (oracle on big shapes)")


def pytest_collection_modifyitems(config, items):
    # GPU tests run last within a session so a CPU failure shows up first.
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)
