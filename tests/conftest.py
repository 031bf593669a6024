import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name: str) -> list:
    """Non-comment lines of a golden fixture, split on whitespace."""
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def golden_map(name: str) -> dict:
    return {r[0]: r[1:] for r in read_golden(name)}


@pytest.fixture(scope="session")
def O():
    from oracle import oracle
    oracle._load()
    return oracle


@pytest.fixture(scope="session")
def S():
    from synth import synth
    synth._load()
    return synth
