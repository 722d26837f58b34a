"""The CPU oracle against the pins (exhaustive, brute-force, closed-form, fixtures)."""

import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    assert pin()
