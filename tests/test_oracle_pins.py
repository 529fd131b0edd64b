"""The oracle against things other than itself (see tests/pins.py for each pin's basis)."""
import pytest

import pins

PINS = [n for n in dir(pins) if n.startswith("pin_")]


@pytest.mark.parametrize("name", PINS)
def test_pin(name):
    getattr(pins, name)()
