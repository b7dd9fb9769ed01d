import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden_bytes(name: str) -> bytes:
    """Parse '<hex offset>: <16 hex bytes>' lines of a golden fixture."""
    out = bytearray()
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            off, data = line.split(":", 1)
            assert int(off, 16) == len(out), (name, off)
            out += bytes(int(b, 16) for b in data.split())
    return bytes(out)
