"""The CPU oracle against its pins (format definitions, brute force, hand-worked examples,
closed forms and invariants).  No GPU and no product code involved."""
import pytest

import oracle_pins as pins
from oracle import nvfp4_ref as ref


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(ref)
