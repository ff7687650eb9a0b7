"""The attention oracle against brute force, torch, closed forms and invariants."""

import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
