"""The fp64 oracle against its pins (CPU only).  See oracle_pins.py."""
import pytest

import os, sys
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from oracle_pins import ALL_PINS  # noqa: E402


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
