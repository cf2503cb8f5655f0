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


def test_bf16_ulp_bound():
    """The comparison's bf16 spacing: 2^-7 relative to the binade."""
    import numpy as np
    from case_oracle import bf16_ulp
    assert bf16_ulp(1.0) == 2.0 ** -7
    assert bf16_ulp(-4.11244) == 2.0 ** -5
    assert bf16_ulp(1.99) == 2.0 ** -7
    assert bf16_ulp(0.3) == 2.0 ** -9
    # -4.11244 lies between the bf16 neighbours -4.125 and -4.09375
    assert abs(-4.125 - -4.11244) < bf16_ulp(-4.11244) and abs(-4.09375 - -4.11244) < bf16_ulp(-4.11244)
