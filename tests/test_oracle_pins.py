"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def libs():
    return oracle._lib("f32"), oracle._lib("f64")


@pytest.mark.parametrize("name", sorted(ALL_PINS))
def test_pin(name, libs):
    ALL_PINS[name](*libs)
