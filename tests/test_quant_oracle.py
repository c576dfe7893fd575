"""The oracle's NVFP4 quantiser against its pins, and the pins against
planted mistakes."""
import pytest

import quant_pins as qp
from oracle import oracle as orc


@pytest.fixture(scope="module")
def o():
    return orc.load()


@pytest.mark.parametrize("pin", qp.ALL_QUANT_PINS, ids=lambda p: p.__name__)
def test_quant_pin(o, pin):
    assert o.mutant == 0
    failures = pin(o)
    assert failures == [], failures[:5]


# planted quantiser mistakes (ORACLE_MUTANT in oracle/nvfp4_oracle.c)
QUANT_MUTANTS = {
    12: "scale truncated instead of rounded to nearest even",
    13: "E2M1 ties away from zero",
    14: "negative values that round to zero lose their sign",
    15: "x times the reciprocal of the scale instead of x / scale",
}


@pytest.mark.parametrize("mutant", sorted(QUANT_MUTANTS), ids=lambda m: QUANT_MUTANTS[m])
def test_quant_pins_catch_planted_mistake(tmp_path, mutant):
    mo = orc.load(orc.build_mutant(mutant, str(tmp_path)))
    assert mo.mutant == mutant
    caught = [p.__name__ for p in qp.ALL_QUANT_PINS if p(mo)]
    assert caught, f"no pin catches mutant {mutant} ({QUANT_MUTANTS[mutant]})"
