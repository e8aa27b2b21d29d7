"""The fp64 oracle against its pins (CPU only)."""

import pytest

import oracle.paged_attention as ora
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(ora)
