"""The fp64 oracle against brute force, closed forms and invariants (CPU only)."""
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)
