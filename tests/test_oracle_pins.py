"""The CPU oracle against its pins (hand tables, library decoders, brute force,
closed forms, invariants). See tests/pins.py for what pins each function."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
