"""The CPU oracle against its pins (closed forms, library special cases,
brute force, finite differences, invariants). Runs without a GPU."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(None)
