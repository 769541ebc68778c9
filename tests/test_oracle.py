"""The CPU oracle against its pins (closed forms, brute force, torch SDPA,
torch's number decoders, hand-derived examples and invariances)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
