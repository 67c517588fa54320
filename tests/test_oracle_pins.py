"""The oracle against what the pages and the mathematics fix (CPU only)."""
import os
import tempfile

import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(oracle_mod, check):
    check(oracle_mod)


# Each planted mistake (see ORACLE_MUTANT in oracle/lora_oracle.c) must be
# caught by at least one pin.
MUTANTS = {
    1: "scale dropped",
    2: "correction subtracted",
    3: "B read transposed",
    4: "A read transposed",
    5: "unstable sort inside an adapter",
    6: "in-page offset dropped",
    7: "none rows take adapter 0",
    8: "last rank term dropped",
    9: "segment length off by one",
    10: "merge ignores coef",
    11: "merge reads A transposed",
    12: "merge drops the scale",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m].replace(" ", "_"))
def test_planted_mistake_is_caught(oracle_mod, mutant):
    with tempfile.TemporaryDirectory() as td:
        path = oracle_mod.build(out=os.path.join(td, "mutant.so"), mutant=mutant)
        oracle_mod.use_library(path)
        caught = []
        try:
            for check in pins.ALL_CHECKS:
                try:
                    check(oracle_mod)
                except AssertionError:
                    caught.append(check.__name__)
        finally:
            oracle_mod.use_library(None)
    assert caught, "planted mistake %r passed every pin" % MUTANTS[mutant]
