"""The CPU oracle against its pins (closed forms, invariants, torch fp64
rms_norm, exact rational brute force, hand-worked golden examples)."""

import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()
