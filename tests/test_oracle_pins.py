"""The oracle against its pins (tests/pins.py): closed forms, brute force, invariants."""

import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)
