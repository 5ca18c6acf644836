"""The comparison metric (oracle/metrics.py) against its pins (tests/metric_pins.py)."""

import pytest

from oracle import metrics
from tests import metric_pins


@pytest.mark.parametrize("pin", metric_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_metric_pin(pin):
    pin(metrics)
