"""The fp64 oracle against its pins (brute force, torch SDPA special cases,
closed forms, invariants).  CPU only."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
