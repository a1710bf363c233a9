"""The CPU oracle against its pins (hand-worked example, library matmuls,
brute force, exact integers, invariants of the definition)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)
