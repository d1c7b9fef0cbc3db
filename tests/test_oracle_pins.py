"""The CPU oracle against its pins (formats, hand-derived goldens, closed
forms, an independent numpy formulation, invariants).  No GPU needed."""

import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(ref, pin):
    pin(ref)
