"""The fp64 oracle, pinned to things other than itself (see pins.py)."""
import pytest

from oracle import oracle as orc_mod
from pins import LIMITS, PINS


@pytest.fixture(scope="module")
def orc():
    orc_mod.build(force=False)
    return orc_mod.Oracle()


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(orc, name):
    err = PINS[name](orc)
    assert err <= LIMITS[name], f"pin {name}: error {err:.3e} > {LIMITS[name]:.1e}"
