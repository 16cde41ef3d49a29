"""The CPU oracle against facts the mathematics fixes (pins K1-K9, stop rule)."""
import pytest

import oracle
import oracle_pins as P


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
