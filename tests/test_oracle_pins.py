"""The CPU oracle against its pins (no GPU)."""
import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    assert orc.mutant == 0
    pin(orc)
