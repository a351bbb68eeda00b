"""Shared pytest setup: the `gpu` marker and on-demand builds.

GPU tests are marked ``@pytest.mark.gpu``; everything else runs on a CPU-only
host.  The oracle library is built here if it is missing (a few seconds of
gcc); the HIP library is only ever loaded, never built, by the tests.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X (gfx950) GPU")


def pytest_sessionstart(session):
    lib = os.path.join(ROOT, "oracle", "liboracle.so")
    if not os.path.exists(lib):
        from oracle import build as obuild
        obuild.build()
