"""The CPU oracle against closed forms, invariants, library routines and brute force."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("check", PINS, ids=[f.__name__ for f in PINS])
def test_pin(orc, check):
    check(orc)
