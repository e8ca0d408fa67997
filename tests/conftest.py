"""Shared fixtures.

GPU tests carry the ``gpu`` marker. On a machine without a HIP device they
skip (the check could not run, which is not a pass); on a machine with one,
a missing HIP library is an error, never a silent fallback.
"""
from __future__ import annotations

import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a HIP device (MI355X) and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle

    return oracle.load()


def _gpu_available() -> bool:
    try:
        import torch
    except ImportError:
        return False
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def cs():
    """The HIP library's Python binding on a device that exists."""
    if not _gpu_available():
        pytest.skip("no HIP device: GPU parity could not be checked here")
    import candidate_scoring_amd

    candidate_scoring_amd.load()  # raises if the library is not built
    return candidate_scoring_amd
