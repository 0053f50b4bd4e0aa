"""The CPU oracle against its pins (closed forms, invariants, golden fixtures, brute force)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)
