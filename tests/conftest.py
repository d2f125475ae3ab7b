"""Shared pytest setup: the ``gpu`` marker and the in-tree libraries.

CPU-only tests (``-m "not gpu"``) cover the generator, the oracle against its
pins, host logic and the C-ABI library's exports.  ``gpu`` tests need an
MI355X and compare the HIP path with the oracle.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950)")


def _ensure_built():
    # the generator and the oracle are plain C built with gcc in seconds;
    # build them only when nothing is built yet
    import oracle
    import synth
    if not os.path.exists(synth.LIB_PATH):
        synth.build()
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()


_ensure_built()


@pytest.fixture(scope="session")
def gpu_available():
    import torch
    return torch.cuda.is_available()
