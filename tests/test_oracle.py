"""The fp64 oracle against its pins (library routine, brute force, closed forms,
invariants from the pages, and the cache write position by position)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)
