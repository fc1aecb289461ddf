"""The CPU oracle against its pins: brute force, library routines, closed forms, hand-built cases."""
import pytest

from . import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle_lib, pin):
    pin(oracle_lib)
