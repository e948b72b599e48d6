"""The CPU oracle against its pins (hand values, closed forms, brute force, library routines)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)
