"""The CPU oracle against its pins (hand-worked examples, library routines,
the pages' printed fragments, brute force and invariants). See
``oracle_pins.py`` for what each pin checks and where it comes from."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)
