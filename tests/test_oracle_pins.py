"""The fp64 oracle against facts fixed outside of it (CPU only)."""
import pytest

import oracle.kmip_oracle as orc
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(orc)
