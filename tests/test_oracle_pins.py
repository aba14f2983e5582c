"""The CPU oracle against its pins (worked examples, library routines, closed
forms and invariants); see oracle_pins.py for what each pin checks."""
import pytest

import oracle_pins
from oracle import ref


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ref.default())
