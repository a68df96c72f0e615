"""The oracle against hand-worked values, closed forms, brute force, torch
library routines and the invariants the pages fix (CPU only)."""
import pytest

import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
