import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


class _Dispatch:
    """Forces the library's launch choice (q2_set_dispatch) for one test; the
    automatic choice is restored afterwards.  Keyword arguments accumulate
    over calls within the test: path, tile, ksplit."""

    def __init__(self, q2):
        self.q2 = q2
        self.state = dict(path=None, tile=None, ksplit=0)

    def __call__(self, **kw):
        unknown = set(kw) - set(self.state)
        if unknown:
            raise TypeError(f"unknown dispatch keys {unknown}")
        self.state.update(kw)
        self.q2.set_dispatch(**self.state)


@pytest.fixture
def force():
    import ternary_weight_quantized_q2_amd as q2
    d = _Dispatch(q2)
    yield d
    q2.set_dispatch(None, None, 0)
