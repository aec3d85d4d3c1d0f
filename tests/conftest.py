import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _print_case(item):
    # Name the case before a GPU step runs, so a run that dies mid-test says which.
    if item.get_closest_marker("gpu") is not None:
        sys.stderr.write("\n[gpu-case] %s\n" % item.nodeid)
        sys.stderr.flush()


def pytest_runtest_setup(item):
    _print_case(item)
