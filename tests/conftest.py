import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def pytest_runtest_setup(item):
    # name the case on stderr before any GPU work starts, so a run that takes
    # the device down still says which test it was in
    if item.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"\n[gpu-test] {item.nodeid}\n")
        sys.__stderr__.flush()
