"""The store-prologue oracle against its pins (tests/rope_pins.py)."""
import pytest

import oracle.store_prologue as rope_oracle
import rope_pins


@pytest.mark.parametrize("check", rope_pins.ALL_CHECKS, ids=[c.__name__ for c in rope_pins.ALL_CHECKS])
def test_rope_pin(check):
    check(rope_oracle)
