"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)
