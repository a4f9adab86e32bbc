"""The oracle against closed forms, brute force, library routines and
hand-built examples (CPU only)."""

import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
