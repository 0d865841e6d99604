"""The float64 oracle against its pins (CPU only)."""

import pytest

from oracle import gdn_oracle as orc

import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(orc)
