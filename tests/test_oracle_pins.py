"""The CPU oracle against its pins (closed forms, invariants, hand-worked fixtures,
brute force).  No GPU."""

import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
