"""The CPU oracle against its pins (no GPU)."""
import pytest

import pins
from oracle import oracle


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
