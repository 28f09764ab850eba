import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The sanitizer pass (tests/test_sanitizers.py) reruns this suite in a child
# process with the AddressSanitizer/UBSan builds of both libraries.
if os.environ.get("KQ_TEST_SANITIZED_LIBS") == "1":
    import oracle as _oracle
    from mxfp4_activation_quantizer_amd import kq as _kq
    _oracle.LIB_PATH = os.path.join(ROOT, "oracle", "libkq_oracle_san.so")
    _kq.LIB_PATH = os.path.join(ROOT, "mxfp4_activation_quantizer_amd", "libkq_san.so")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")
    config.addinivalue_line("markers", "sanitize: runs the CPU suite under the sanitizers")


@pytest.fixture(scope="session")
def oracle():
    import oracle as o
    o.lib()
    return o
