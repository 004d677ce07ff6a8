"""Shared test setup: the ``gpu`` marker, and building the CPU oracle.

Tests marked ``gpu`` need a real MI355X and the built ``libgsraster.so``;
everything else runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _oracle_stale():
    lib = os.path.join(ROOT, "oracle", "liboracle.so")
    src = os.path.join(ROOT, "oracle", "oracle.cpp")
    return (not os.path.exists(lib)) or os.path.getmtime(lib) < os.path.getmtime(src)


@pytest.fixture(scope="session", autouse=True)
def _build_oracle():
    if _oracle_stale():
        import oracle
        oracle.build(force=True)
    yield
