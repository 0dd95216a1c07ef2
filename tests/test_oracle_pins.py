"""CPU tier: the oracle against its pins (see tests/pins.py for each source)."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ALL, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
