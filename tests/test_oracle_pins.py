"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def ora():
    return oracle.default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin, ora):
    pin(ora)
