"""The oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins as P


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("name", P.golden_files())
def test_golden(orc, name):
    P.pin_golden(orc, name)


@pytest.mark.parametrize("pin", [p for p in P.ALL_PINS if p is not P.pin_all_golden], ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
