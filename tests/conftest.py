import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the C ABI on the GPU)")


def golden_rows(name):
    """Non-comment, non-empty rows of a golden fixture, split on whitespace."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def tsl_lib():
    """The built C-ABI library through its binding (builds it when absent)."""
    from tensor_sharded_linear_plan_amd import build as tbuild
    if not os.path.exists(tbuild.LIBRARY):
        tbuild.build()
    from tensor_sharded_linear_plan_amd import binding
    return binding
