"""The CPU oracle against its pins (see oracle_pins.py for what each fixes)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle._get_lib())


def test_oracle_threads():
    assert oracle.num_threads() >= 1
