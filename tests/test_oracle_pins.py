"""The CPU oracle against its pins (no GPU needed)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
