"""The fp64 oracle against what the pages and mathematics fix (CPU only)."""
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)
