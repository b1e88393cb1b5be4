import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


def load_golden(name):
    """Parse a golden fixture: '# ...' comments, then 'key v1 v2 ...' lines.
    Repeated keys accumulate into a list of rows."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            vals = [float(v) for v in vals]
            if key in out:
                if not isinstance(out[key][0], list):
                    out[key] = [out[key]]
                out[key].append(vals)
            else:
                out[key] = vals
    return out


@pytest.fixture
def golden():
    return load_golden
