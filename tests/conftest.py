import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large-size case (minutes)")


def pytest_collection_modifyitems(config, items):
    # Run GPU tests in file order but after the CPU tests of the same session.
    items.sort(key=lambda it: 1 if it.get_closest_marker("gpu") else 0)
