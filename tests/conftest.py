import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def orc():
    """The oracle: the default build, or the build SPECVERIFY_ORACLE names
    (the sanitizer runs use an instrumented one)."""
    import oracle
    path = os.environ.get("SPECVERIFY_ORACLE")
    return oracle.Oracle(path) if path else oracle.default()
