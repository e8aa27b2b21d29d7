"""The fp64 oracle against its pins (CPU only)."""

import pytest

import oracle.paged_attention as ora
import oracle.sinks_window as sw
from tests.oracle_pins import ALL_PINS
from tests.oracle_pins_sinks import SINK_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(ora)


@pytest.mark.parametrize("pin", SINK_PINS, ids=lambda p: p.__name__)
def test_sinks_window_pin(pin):
    pin(sw)
