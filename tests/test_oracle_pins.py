"""The oracle against its pins (hand-worked examples, torch CPU float64,
autograd, format invariants, special cases, brute force)."""
import pytest

import oracle
from oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(oracle)
