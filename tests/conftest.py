import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (full-size stream) case")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture
def golden():
    import json

    def load(name):
        with open(os.path.join(GOLDEN, name)) as f:
            return json.load(f)
    return load


# A host-sanitizer run of the CPU tests loads an instrumented build of the library
# instead of the in-tree one (tests/test_host_sanitizers.py sets this variable in the
# child process it starts).
if os.environ.get("LA_TEST_LIB_PATH"):
    from streaming_causal_video_amd import _lib as _la_lib
    _la_lib.LIB_PATH = os.environ["LA_TEST_LIB_PATH"]
