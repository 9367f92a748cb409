import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libkvdecode.so")


def golden_path(name: str) -> str:
    return os.path.join(GOLDEN, name)


@pytest.fixture(scope="session")
def golden():
    import json

    def load(name):
        with open(golden_path(name)) as f:
            return json.load(f)
    return load
