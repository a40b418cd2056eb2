import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: a CPU test that takes more than a few seconds")


def pytest_runtest_setup(item):
    # Name the case before it runs, so a run that ends abruptly still says where it was.
    if item.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-case] {item.nodeid}", flush=True)
