"""Shared pytest set-up: the ``gpu`` marker and the CPU-side libraries.

CPU tests (``-m "not gpu"``) cover the oracle against its pins, the input
generator, host logic and the C-ABI library's exports.  GPU tests (``-m gpu``)
compare the HIP path with the oracle through the C-ABI.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session", autouse=True)
def _cpu_libraries():
    """Build the generator and oracle libraries if this tree has none yet."""
    import oracle
    import synthetic_inputs
    synthetic_inputs.build(force=False)
    oracle.build(force=False)
    yield
