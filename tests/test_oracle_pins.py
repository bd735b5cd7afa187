"""The fp64 oracle against closed forms, invariants, SDPA and brute force."""

import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
