"""The CPU oracle against its pins (page values, closed forms, invariants)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_pin(oracle, pin):
    pin(oracle)
