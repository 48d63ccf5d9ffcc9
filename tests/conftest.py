"""Shared pytest setup: the `gpu` marker and import paths.

Tests marked ``gpu`` need a ROCm GPU and the built HIP library; everything else
runs on the CPU (oracle pins, generator checks, host-side library checks).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a ROCm GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle._load()
    return oracle


@pytest.fixture(scope="session")
def synth_mod():
    import synth
    synth._load()
    return synth
