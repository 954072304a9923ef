"""The CPU oracle against its pins (hand-worked example, brute force, numpy
dense attention, closed forms, invariants)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
