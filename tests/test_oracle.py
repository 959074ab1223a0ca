"""The fp64 oracle against its pins (library routines, closed forms, invariants)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)
