"""The ParisKV-style retrieval oracle against its pins (CPU only)."""
import pytest

from oracle import paris
from paris_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(paris)
