"""The CPU oracle against its pins (see oracle_pins.py for what each pins it to)."""

import pytest

import oracle_pins as P


@pytest.fixture(scope="module")
def orc(oracle_lib):
    return oracle_lib


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_pin(orc, pin):
    pin(orc)
