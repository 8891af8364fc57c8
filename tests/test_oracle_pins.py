"""The CPU oracle against its pins (closed forms, exact integer and rational
arithmetic, special matrices, numpy's fp64 matmul, invariants)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)
