"""Shared pytest set-up: the ``gpu`` marker and import paths.

Tests marked ``gpu`` need a HIP device and the built HIP library; everything
else runs on the CPU (oracle pins, host-side argument checks, symbol exports).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a HIP GPU (MI355X) and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


def read_golden(name):
    """Lines of a golden fixture with comments and blank lines removed."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line)
    return out
