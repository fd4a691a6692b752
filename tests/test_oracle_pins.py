"""The CPU oracle against its pins (no GPU)."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(oracle, pin):
    assert oracle.mutant == 0
    pin(oracle)
