"""The CPU oracle against its pins (hand-worked values, closed forms,
identities, library routines, PIVOT invariants). No GPU."""
import pytest

import oracle
from pins import ALL_PINS


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin, lib):
    pin(lib)
