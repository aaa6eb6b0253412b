import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a 'key v1 v2 ...' fixture; '#' lines are comments. Hex tokens are ints."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            parsed = []
            for v in vals:
                if v.startswith("0x"):
                    parsed.append(int(v, 16))
                else:
                    try:
                        parsed.append(int(v))
                    except ValueError:
                        try:
                            parsed.append(float(v))
                        except ValueError:
                            parsed.append(v)
            out.setdefault(key, []).append(parsed)
    return {k: (v[0] if len(v) == 1 else v) for k, v in out.items()}


@pytest.fixture
def golden():
    return read_golden
