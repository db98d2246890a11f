"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle_pins as pins
from oracle import crisp_oracle as co
from oracle import driver

CHECKS = [name for name in dir(pins) if name.startswith("check_")]
DRIVER_CHECKS = [name for name in dir(pins) if name.startswith("dcheck_")]


@pytest.mark.parametrize("name", CHECKS)
def test_pin(name):
    getattr(pins, name)(co)


@pytest.mark.parametrize("name", DRIVER_CHECKS)
def test_driver_pin(name):
    getattr(pins, name)(driver)
