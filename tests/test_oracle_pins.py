"""The oracle against its pins (closed forms, invariants, library routines and
the pages' printed values); CPU only."""

import pytest

from oracle import infini_ref
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(infini_ref)
