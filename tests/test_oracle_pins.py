"""The fp64 oracle against its pins (closed forms, brute force, library special cases, invariants, hand example)."""
import pytest

from oracle import prr_oracle
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(prr_oracle)
