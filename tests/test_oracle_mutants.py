"""Each planted mistake in the oracle must be caught by at least two pins.

The oracle source carries twenty compile-time mutants (a dropped term, a wrong
sign, an off-by-one, a transposed operand, ...).  Building each one and
running the pins shows that the pins constrain every step of the oracle.
"""

import pytest

import oracle
import oracle_pins

MUTANTS = {
    1: "ties ordered by descending index",
    2: "ReLU dropped",
    3: "page and slot transposed",
    4: "tail omitted",
    5: "one indexer head dropped",
    6: "softmax scale dropped",
    7: "a repeated index counted once",
    8: "visible-block rule off by one",
    9: "a hole read as token 0",
    10: "scores ordered ascending",
    11: "fp8 key scale ignored",
    12: "e4m3 exponent bias 8",
    13: "e4m3 subnormal read as normal",
    14: "head weights ignored",
    15: "ReLU after the head weight",
    16: "top-k per row reads past the visible blocks",
    17: "a request's first token given to the request before",
    18: "logical positions counted from the sequence end",
    19: "compressed slot written at a group's first token",
    20: "no k work item without a completed group",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m].replace(" ", "_"))
def test_mutant_is_caught(tmp_path, mutant):
    path = oracle.build(str(tmp_path / f"liboracle_m{mutant}.so"), mutant=mutant)
    orc = oracle.Oracle(path)
    assert orc.mutant == mutant
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
            if len(caught) == 2:
                break
    assert len(caught) >= 2, f"mutant {mutant} ({MUTANTS[mutant]}) caught only by {caught}"
