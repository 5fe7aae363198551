"""The fp64 oracle against its pins (closed forms, textbook special cases,
brute force, finite differences, invariants); CPU only."""
import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(ora, name):
    PINS[name](ora)
