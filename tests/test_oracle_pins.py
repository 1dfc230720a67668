"""The oracle against its pins (CPU only)."""
import pytest

from oracle import bsga_oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(bsga_oracle)
