"""The CPU oracle against the pins in tests/pins.py (no GPU)."""
import pytest

import oracle.moe_oracle as O
import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(O)
