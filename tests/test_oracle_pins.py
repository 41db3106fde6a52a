"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("name", sorted(oracle_pins.ALL_PINS))
def test_pin(orc, name):
    oracle_pins.ALL_PINS[name](orc)
