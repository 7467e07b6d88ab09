"""The oracle against its pins (hand-worked values, closed forms, library
routines, brute-force definitions). CPU only."""
import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)
