"""Shared pytest configuration.

Markers:
  gpu -- needs an AMD MI355X (gfx950) and the built libnq.so; everything else
         runs on a CPU-only host.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (built on first use)."""
    import oracle
    oracle.lib()
    return oracle
