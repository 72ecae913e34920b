"""The CPU oracle against closed forms, invariants, brute force, torch SDPA and the pages' numbers."""

import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
