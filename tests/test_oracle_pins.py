"""The CPU oracle against the facts that pin it (see tests/pins.py)."""
import pytest

import pins

pytestmark = pytest.mark.cpu


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
