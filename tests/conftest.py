import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# A sanitized build under test (tests/test_sanitizers.py runs the host tests
# in a subprocess with these set): the binding loads the library from
# LORA_TEST_LIB_DIR, the oracle tests load the oracle from LORA_TEST_ORACLE_LIB.
if os.environ.get("LORA_TEST_LIB_DIR"):
    import lora_row_adapter_amd._binding as _b
    _b._HERE = os.environ["LORA_TEST_LIB_DIR"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU case")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    if os.environ.get("LORA_TEST_ORACLE_LIB"):
        oracle.use_library(os.environ["LORA_TEST_ORACLE_LIB"])
        return oracle
    oracle.build(force=not os.path.exists(os.path.join(ROOT, "oracle", "liblora_oracle.so")))
    oracle.use_library(None)
    return oracle
