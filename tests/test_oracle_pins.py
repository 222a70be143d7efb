"""The fp64 oracle against hand-worked values, closed forms, invariants, a
library routine and a brute force (see oracle_pins.py for each pin)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(oracle.lora_oracle)
