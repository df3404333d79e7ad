"""pytest configuration: the `gpu` marker and the repository root on sys.path."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built HIP library")


@pytest.fixture
def knobs():
    """knobs(name, value): override a library tuning knob for this test (restored afterwards;
    value -1 restores the default at once)."""
    tq = pytest.importorskip("moe_expert_ffn_q4_amd")
    changed = {}

    def set_knob(name, value):
        if name not in changed:
            changed[name] = tq.get_knob(name)
        tq.set_knob(name, int(value))

    yield set_knob
    for name, value in changed.items():
        tq.set_knob(name, value)
