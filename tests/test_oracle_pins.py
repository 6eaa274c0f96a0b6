"""The CPU oracle against closed forms, library routines, hand-derived fixtures and
brute force (see oracle_pins.py)."""

import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.lsa_ref)

