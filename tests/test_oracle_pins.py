"""The CPU oracle against its pins (exact-rational brute force, closed forms,
an independent binary64 route, torch's bf16 conversion, invariants and error
bounds).  No GPU."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)
