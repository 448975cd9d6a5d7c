"""The CPU oracle against its pins (worked example, library routines, brute force,
closed forms, invariants).  CPU only."""

import pytest

import oracle
from pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)
