"""The CPU oracle against its pins (closed forms, independent codecs, exact sums, page values)."""

import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)
