"""The chunked-prefill oracle against values fixed by the pages and by
mathematics."""
import pytest

import oracle
from tests import prefill_pins as P


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda p: p.__name__)
def test_pin_holds(orc, pin):
    assert pin(orc) is None


MUTANTS = {
    8: "no causal mask inside the chunk",
    9: "causal mask off by one (own position excluded)",
    3: "q-head -> kv-head map h % Hkv (shared with decode)",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: MUTANTS[m])
def test_mutant_is_caught(mutant):
    fails = P.failures(oracle.build_mutant(mutant))
    assert fails, f"mutant {mutant} ({MUTANTS[mutant]}) passed every prefill pin"
