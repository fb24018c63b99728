import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_report_header(config):
    """Name the library under test by its source digest; loading refuses a library built from other
    sources than the working tree's (a stale build), which ends the session here."""
    from activation_sparse_moe_amd import _capi, build
    if not os.path.exists(_capi.LIB_PATH):
        return f"libblockffn: not built (sources {build.library_digest()})"
    try:
        return f"libblockffn: {_capi.LIB_PATH}, built from sources {_capi.build_digest()}"
    except RuntimeError as e:
        raise pytest.UsageError(str(e))


@pytest.fixture(scope="session")
def golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "hand_examples.json")) as f:
        return json.load(f)
