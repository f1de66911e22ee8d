"""The row-reduction oracle (oracle/rows.py) against its pins (CPU only)."""

import pytest

import rows_pins
from oracle import rows as R


@pytest.mark.parametrize("pin", rows_pins.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(R)
