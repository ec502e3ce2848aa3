"""The fp64 oracle against closed forms, invariants, library routines and the
hand-derived worked example (CPU only)."""
import pytest

from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(oracle, pin):
    pin(oracle)
