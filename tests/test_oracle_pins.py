"""The oracle checked against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
