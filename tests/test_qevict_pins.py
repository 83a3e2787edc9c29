"""The window-routed (QEvict-form) oracle against its pins (CPU only)."""
import pytest

from oracle import qevict
from qevict_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(qevict)
