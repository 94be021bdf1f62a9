import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU-only check")


@pytest.fixture(scope="session")
def grids_compact():
    import synth
    return synth.grid_compact(synth.QTYPE_IQ2XS), synth.grid_compact(synth.QTYPE_IQ1M)


@pytest.fixture(scope="session")
def ogrids(grids_compact):
    import oracle
    return oracle.grids(*grids_compact)
