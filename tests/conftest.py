import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    """The tests load the in-tree built libraries; build whichever is missing (once, here) so
    that a fresh checkout tests without a separate build step.  Nothing is rebuilt if present."""
    from attention_fa_fwd_amd import build

    if not os.path.exists(build.LIB_PATH):
        build.build_library(verbose=True)
    if not os.path.exists(build.PROBE_PATH):
        build.build_probe(verbose=True)
    if not os.path.exists(build.C_CALLER_BIN):
        build.build_c_caller(verbose=True)
