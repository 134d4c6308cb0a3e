"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
from tests.pins import ALL_PINS


@pytest.mark.parametrize("name", sorted(ALL_PINS))
def test_oracle_pin(name):
    ALL_PINS[name](oracle.load())
