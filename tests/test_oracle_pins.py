"""The fp64 oracle against the pins (CPU only)."""
import pytest

import oracle
from oracle_pins import ALL_PINS, BWD_PINS, EPI_PINS, SLSTM_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.mark.parametrize("pin", ALL_PINS + BWD_PINS + EPI_PINS + SLSTM_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
