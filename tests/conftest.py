import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def golden_path(name: str) -> str:
    return os.path.join(ROOT, "tests", "golden", name)


def read_fixture(name: str) -> dict:
    """Parse a `key v1 v2 ...` fixture, skipping comment lines."""
    out = {}
    with open(golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def hexbytes(vals) -> bytes:
    return bytes(int(v, 16) for v in vals)
