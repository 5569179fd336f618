"""The fp64 oracle against the pages' worked example, closed forms, scipy and
a 50-digit brute force (CPU only)."""
import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()
