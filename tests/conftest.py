"""Shared pytest setup: the repo root on sys.path and the ``gpu`` marker.

Tests marked ``gpu`` need an MI355X and the built HIP library; everything else
runs on the CPU (``pytest -m "not gpu"``).
"""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


import json

import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture
def golden():
    """Load a JSON fixture from tests/golden (values printed on the pages)."""

    def load(name):
        with open(os.path.join(GOLDEN, name)) as f:
            return json.load(f)

    return load
