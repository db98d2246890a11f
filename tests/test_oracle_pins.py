"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle_pins as pins
from oracle import crisp_oracle as co

CHECKS = [name for name in dir(pins) if name.startswith("check_")]


@pytest.mark.parametrize("name", CHECKS)
def test_pin(name):
    getattr(pins, name)(co)
