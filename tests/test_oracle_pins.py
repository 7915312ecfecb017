"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""

import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()
