import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def parse_mask_golden(path):
    """Parse tests/golden/masks_8x8.txt into {name: (params, 0/1 rows)}."""
    out, name, params, rows = {}, None, None, []
    with open(path) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("name "):
                if name:
                    out[name] = (params, rows)
                name, params, rows = line.split()[1], None, []
            elif line.startswith("params "):
                params = dict(kv.split("=") for kv in line.split()[1:])
                params = {k: int(v) for k, v in params.items()}
            else:
                rows.append([1 if ch == "1" else 0 for ch in line])
    if name:
        out[name] = (params, rows)
    return out


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
