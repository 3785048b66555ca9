"""The oracle against its pins (CPU only). See oracle_pins.py for what each pin fixes."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def ref():
    return oracle.default()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(ref, pin):
    pin(ref)
