import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (run through the HIP library)")
    config.addinivalue_line("markers", "slow: large CPU build; skipped unless selected")
    import helpers
    helpers.CAPTURE = config.pluginmanager.getplugin("capturemanager")


@pytest.fixture(scope="session")
def worked_example():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    return oracle


@pytest.fixture(scope="session")
def synth_mod():
    from grammar_compressed_sparse_amd import synth
    return synth
