"""The bounds of ``oracle/bounds.py`` against inputs that nearly reach them
(``tests/pins_bounds.py``), and planted changes: each test below copies
``bounds.py``, doubles one main term or drops the second term of bound (1),
loads the copy as a module and checks that at least one pin fails on it.
No GPU."""
import importlib.util
import os

import pytest

import oracle
import pins_bounds
from oracle import bounds

BOUNDS_SRC = os.path.join(os.path.dirname(oracle.__file__), "bounds.py")

MUTANTS = {
    "requant_scale_term_doubled": ("return s_elem / 2.0 + 2.0 ** -22 * x_abs + 2 * TINY",
                                   "return s_elem + 2.0 ** -22 * x_abs + 2 * TINY"),
    "requant_second_term_dropped": ("return s_elem / 2.0 + 2.0 ** -22 * x_abs + 2 * TINY",
                                    "return s_elem / 2.0 + 2 * TINY"),
    "oneshot_output_term_doubled": ("bound += per_element(scale_out, block, n) / 2.0 + 2.0 ** -22",
                                    "bound += per_element(scale_out, block, n) + 2.0 ** -22"),
    "ring_scale_term_doubled": ("b += per_element(s, block, n) / 2.0 + 2.0 ** -21",
                                "b += per_element(s, block, n) + 2.0 ** -21"),
    "e4m3_relative_term_doubled": ("E4M3_REL = 2.0 ** -4 + 4 * U", "E4M3_REL = 2.0 ** -3 + 8 * U"),
    "e4m3_absolute_term_doubled": ("E4M3_ABS = 2.0 ** -10 + U", "E4M3_ABS = 2.0 ** -9 + 2 * U"),
}


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.mark.parametrize("pin", pins_bounds.PINS, ids=lambda p: p.__name__)
def test_bounds_pin(pin, o):
    pin(bounds, o)


def _mutant_module(old: str, new: str, tmp_path):
    src = open(BOUNDS_SRC).read()
    assert src.count(old) == 1, old
    path = tmp_path / "bounds_mutant.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("bounds_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_change_is_caught(name, o, tmp_path):
    mod = _mutant_module(*MUTANTS[name], tmp_path)
    failed = []
    for pin in pins_bounds.PINS:
        try:
            pin(mod, o)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin fails with {name}"
