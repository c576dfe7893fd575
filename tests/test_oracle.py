"""The CPU oracle against its pins, and the pins against planted mistakes."""
import pytest

import oracle_pins as pins
from oracle import oracle as orc


@pytest.fixture(scope="module")
def o():
    return orc.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(o, pin):
    assert o.mutant == 0
    failures = pin(o)
    assert failures == [], failures[:5]


# Each planted mistake (see ORACLE_MUTANT in oracle/nvfp4_oracle.c):
MUTANTS = {
    1: "nibble order swapped",
    2: "E4M3 subnormal scales flushed to zero",
    3: "E2M1 sign dropped",
    4: "one scale per 32 elements instead of 16",
    5: "B read as a transposed (K/2 x N) operand",
    6: "alpha ignored",
    7: "E4M3 exponent bias off by one",
    8: "wrong largest E2M1 magnitude",
    9: "fp32 accumulation",
    10: "truncation instead of round-to-nearest-even",
    11: "sum of products instead of sum of magnitudes for the tolerance",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m])
def test_pins_catch_planted_mistake(tmp_path, mutant):
    lib = orc.build_mutant(mutant, str(tmp_path))
    mo = orc.load(lib)
    assert mo.mutant == mutant
    results = pins.run_all(mo, quick=True)
    caught = [name for name, fails in results.items() if fails]
    assert caught, f"no pin catches mutant {mutant} ({MUTANTS[mutant]})"
