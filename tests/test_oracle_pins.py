"""The fp64 oracle against closed forms, invariants and brute force."""
import pytest

import oracle
import oracle_pins

PINS = oracle_pins.ALL_PINS


@pytest.fixture(scope="module")
def O():
    return oracle.get()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(O, pin):
    pin(O)
