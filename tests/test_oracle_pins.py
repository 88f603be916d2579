"""The CPU oracle against the pages' worked numbers, closed forms, brute force and
independent library routes (see tests/oracle_pins.py for each pin's statement)."""
import pytest

from tests.oracle_pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(orc, name):
    PINS[name](orc)
