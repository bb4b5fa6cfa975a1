import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU check, run only when ZERO_EXHAUSTIVE=1")


def pytest_collection_modifyitems(config, items):
    if os.environ.get("ZERO_EXHAUSTIVE") == "1":
        return
    skip = pytest.mark.skip(reason="exhaustive check: set ZERO_EXHAUSTIVE=1")
    for it in items:
        if "slow" in it.keywords:
            it.add_marker(skip)


def golden_rows(name):
    """Non-comment, non-empty lines of a golden fixture, split on whitespace."""
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows
