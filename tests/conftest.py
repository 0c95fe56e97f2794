import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built library")


def bits_of(x):
    """float array -> bfloat16 bit patterns (round to nearest even)."""
    import numpy as np
    from synthetic import round_to_bf16_bits
    return round_to_bf16_bits(np.asarray(x, dtype=np.float32))


@pytest.fixture
def rng():
    import numpy as np
    return np.random.Generator(np.random.PCG64(1234))
