"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__[4:])
def test_pin(orc, pin):
    pin(orc)
