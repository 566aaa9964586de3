import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Rows of a golden fixture, '#' comment lines dropped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def gpu():
    """The HIP library, loaded; GPU tests fail (not skip) when the library is
    missing on a machine that has a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import bit_quantized_kv_rotate_amd as kvq
    kvq.library()          # raises if libkvq.so is missing or stale
    return kvq
