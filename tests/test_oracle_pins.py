"""The CPU oracle against library routines, brute force, invariants and special cases."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
