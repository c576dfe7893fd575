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


def _wrong_grouped_weights(o):
    """Grouped GEMM that gives each group the next group's weights."""
    import numpy as np

    def f(ac, as_, bc, bs, offsets, alpha):
        G = bc.shape[0]
        return o.grouped_gemm(ac, as_, np.roll(bc, 1, axis=0), np.roll(bs, 1, axis=0), offsets, alpha)
    return f


def _wrong_grouped_rows(o):
    """Grouped GEMM whose row ranges are shifted by one row."""
    import numpy as np

    def f(ac, as_, bc, bs, offsets, alpha):
        M = ac.shape[0]
        off = np.minimum(np.asarray(offsets) + 1, M)
        off[0] = 0
        return o.grouped_gemm(ac, as_, bc, bs, off, alpha)
    return f


@pytest.mark.parametrize("wrong", [_wrong_grouped_weights, _wrong_grouped_rows],
                         ids=["weights of another group", "row ranges off by one"])
def test_grouped_pin_catches_planted_mistake(o, wrong):
    assert pins.pin_grouped_bruteforce(o, cases=60, grouped=wrong(o)), "pin missed the mistake"
