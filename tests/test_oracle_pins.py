"""The fp64 oracle against what the pages and mathematics fix (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load(oracle.LIB)


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)
