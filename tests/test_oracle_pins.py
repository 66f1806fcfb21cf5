"""The oracle against its pins (CPU only)."""
import pytest

import oracle_pins
from oracle import oracle as O


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O.lib())
