"""The CPU oracle against its pins (hand-worked fixtures, exact rationals,
torch's bf16 cast, closed-form invariants).  See oracle_pins.py."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)
