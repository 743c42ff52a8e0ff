import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size GPU parity case (seconds to a minute)")


import pytest  # noqa: E402


@pytest.fixture
def tune():
    """Sets library tuning knobs for one test (tune(decode_chunk=512, ...)) and
    restores their previous values afterwards."""
    import exact_attention_31_amd as E
    saved = {}

    def set_knobs(**knobs):
        for name, value in knobs.items():
            old = E.set_tuning(name, int(value))
            saved.setdefault(name, old)

    yield set_knobs
    for name, value in saved.items():
        E.set_tuning(name, value)
