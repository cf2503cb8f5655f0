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


def test_compare_bracket_only_from_four():
    """The one exception to max|err| <= 1e-2: at |ref| >= 4 an output may be
    either bf16 neighbour of the exact value; below 4 the plain bar holds."""
    import numpy as np
    import pytest as _pt
    from case_oracle import bf16_bracket, compare
    lo, hi = bf16_bracket(np.array([-4.11244, 2.23167, 5.0]))
    assert lo[0] == -4.125 and hi[0] == -4.09375
    assert lo[1] == 2.21875 and hi[1] == 2.234375
    assert lo[2] == hi[2] == 5.0
    compare(np.array([-4.125]), np.array([-4.11244]), "nearest neighbour at |ref| >= 4")
    compare(np.array([-4.09375]), np.array([-4.11244]), "farther neighbour at |ref| >= 4")
    compare(np.array([2.234375]), np.array([2.23167]), "correctly rounded below 4")
    with _pt.raises(AssertionError):  # a neighbour below 4 that misses 1e-2 fails
        compare(np.array([2.21875]), np.array([2.23167]), "farther neighbour below 4")
    with _pt.raises(AssertionError):  # two steps away at |ref| >= 4 fails
        compare(np.array([-4.15625]), np.array([-4.11244]), "two bf16 steps away")

