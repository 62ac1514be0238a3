"""The CPU oracle against its pins (exact-rational brute force, closed forms,
an independent binary64 route, torch's bf16 and float8_e4m3fn conversions,
invariants and error bounds).  No GPU."""
import pytest

import pins
import pins_e4m3
import pins_int4


@pytest.mark.parametrize("pin", pins.ALL_PINS + pins_e4m3.ALL_PINS + pins_int4.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)
