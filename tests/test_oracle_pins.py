"""The CPU oracle against hand-worked values from the pages, library routines, brute-force
element loops and invariants (no GPU)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(oracle)
