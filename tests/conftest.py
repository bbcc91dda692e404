"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X and the in-tree HIP library; everything else
runs on the CPU (oracle pins, host-side argument checks, symbol exports)."""
from __future__ import annotations

import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X GPU")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    oracle.build(force=False)
    return oracle


@pytest.fixture(scope="session")
def nthreads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 1
