import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    """The oracle is plain C built with gcc in about a second; build it when a
    fresh checkout lacks it so the CPU suite runs anywhere."""
    from oracle import LIB_PATH
    if not os.path.exists(LIB_PATH):
        from oracle.build import build
        build()
    yield


@pytest.fixture
def set_knob():
    """set_knob(which, value): a library test override (tfla_dbg_set_knob)
    for this test only; every knob it touched is cleared afterwards."""
    from mlstm_sequence_amd import tfla
    touched = []

    def _set(which, value):
        tfla.tfla_dbg_set_knob(which, int(value))
        touched.append(which)

    yield _set
    for which in touched:
        tfla.tfla_dbg_set_knob(which, -1)
