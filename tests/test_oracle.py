"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_oracle_threads():
    assert oracle.num_threads() >= 1
