"""Each deliberate mistake planted in a copy of the oracle (the MUTANT sites
of oracle/sq_oracle.c) must be caught by at least one pin (CPU only)."""
import pytest

import oracle
import pins

MUTANTS = {
    1: "rounds halves away from zero",
    2: "no 1e-8 floor on the row max",
    3: "token and channel scales swapped in the dequant",
    4: "weight exponent alpha instead of 1 - alpha",
    5: "multiplies activations by s",
    6: "weight column max without abs",
    8: "weight operand read transposed",
    9: "bias dropped",
    10: "row max divided by 128",
    12: "powers multiplied instead of divided",
    13: "calibration max without abs",
    14: "per-tensor scale floored instead of replaced by 1",
    15: "per-tensor max divided by 128",
    16: "weight-only linear scaled by the token index",
    17: "weight-only linear drops the bias",
    18: "reference linear drops the last k term",
    19: "relative error measured against y_q",
    20: "general-alpha power with base and exponent swapped",
    21: "general-alpha power with the complementary exponent",
    22: "alpha = sigmoid(-eta)",
    23: "straight-through weight gradient with the wrong token's scale",
    24: "X / s differentiated as X * s",
    25: "the floor of s passes the gradient everywhere",
    26: "the sigmoid's derivative left out of deta",
    27: "auxiliary loss gradient without the factor 2",
}


@pytest.mark.parametrize("n", sorted(MUTANTS), ids=lambda n: f"m{n}")
def test_mutant_is_caught(n, tmp_path):
    o = oracle.mutant(n, str(tmp_path))
    assert o.mutant == n
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, OverflowError):
            caught.append(pin.__name__)
    assert caught, f"mutant {n} ({MUTANTS[n]}) passes every pin"
