"""The CPU oracle against hand-worked examples, closed forms, library routines and
brute force (see tests/oracle_pins.py for what each check fixes)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(oracle)
