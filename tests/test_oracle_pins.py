"""The CPU oracle against its pins (worked example, closed forms, library
routine, invariants, tiled-method algebra).  CPU only."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
