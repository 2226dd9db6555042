import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


@pytest.fixture(scope="session")
def golden():
    import json
    out = {}
    gdir = os.path.join(HERE, "golden")
    for name in os.listdir(gdir):
        if name.endswith(".json"):
            with open(os.path.join(gdir, name)) as f:
                out[name[:-5]] = json.load(f)
    return out
