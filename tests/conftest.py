import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger oracle runs")


def _flush_name(item):
    # Name the case before it touches the GPU, so a run that dies mid-test
    # still says which case it was.
    if item.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-case] {item.nodeid}", flush=True)


@pytest.hookimpl(tryfirst=True)
def pytest_runtest_setup(item):
    _flush_name(item)
