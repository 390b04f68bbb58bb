"""The fp64 oracle against its pins (facts fixed by the pages and by
mathematics); see oracle_pins.py for each pin and its source."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    oracle.build.build()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
