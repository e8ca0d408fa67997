"""The oracle against what the page and the mathematics fix (CPU only)."""
import pytest

from pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)
