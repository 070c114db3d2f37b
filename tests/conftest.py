import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")

# Another build of the same library (the host-sanitized one of
# test_host_sanitizers.py) may stand in for lib/libiq.so.
if os.environ.get("IQ_TEST_LIBRARY"):
    from compressed_space_attention_isoquant_amd import binding as _binding
    _binding.LIB_PATH = os.environ["IQ_TEST_LIBRARY"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture
def golden():
    return load_golden
