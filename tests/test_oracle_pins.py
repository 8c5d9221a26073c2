"""The CPU oracle against its pins (hand-worked answers, library routines, closed forms, invariants)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)
