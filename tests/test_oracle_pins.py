"""The fp64 oracle against its pins (closed forms, invariants, brute force,
exact rationals, the hand-worked golden example).  CPU only."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
