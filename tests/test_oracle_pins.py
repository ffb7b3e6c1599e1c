"""The CPU oracle against its pins (what the pages and the mathematics fix)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def O():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(O, pin):
    pin(O)
