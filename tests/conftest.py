"""Shared test set-up: repo root on sys.path, the `gpu` marker, and helpers.

Tests marked `gpu` need an MI355X and the built HIP library; everything else
runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def oracle():
    import oracle as O
    O._load()
    return O
