"""The CPU oracle checked against what the paper and mathematics fix (CPU only)."""
import pytest

import oracle.retopk_oracle as O
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(O)
