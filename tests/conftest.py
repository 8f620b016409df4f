import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle work that takes more than a few seconds on the CPU")


@pytest.fixture
def set_knobs():
    """set_knobs(split_ctas=..., pair_cols=..., no_skinny=..., spin_limit=...)
    sets the library's launch knobs for one test; the defaults come back
    after it."""
    from ternary_weight_quantization_amd import binding as B

    yield B.bitnet_set_test_knobs
    B.bitnet_set_test_knobs()
