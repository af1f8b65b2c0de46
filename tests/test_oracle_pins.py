"""The CPU oracle against its pins (hand-derived fixtures, closed forms, invariants)."""
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.Oracle())
