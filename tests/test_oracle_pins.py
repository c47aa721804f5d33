"""The CPU oracle against its pins (closed forms, invariants, printed offsets, brute force)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.mark.parametrize("name,pin", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_pin(orc, name, pin):
    pin(orc)
