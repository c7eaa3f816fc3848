"""Shared pytest configuration.

Tests marked ``gpu`` call the HIP library through its C-ABI and need an MI355X;
everything else runs on the CPU (oracle pins, host metadata, symbol exports).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def repo_root():
    return ROOT
