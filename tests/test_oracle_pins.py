"""The oracle against facts outside itself (see oracle_pins.py)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(__file__))

import oracle as O

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(O)
