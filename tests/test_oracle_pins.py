"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
from pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.default())
