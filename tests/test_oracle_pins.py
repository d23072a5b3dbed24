"""The CPU reference against its pins (closed forms, invariants, library routines,
brute force).  CPU only."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__[6:])
def test_oracle_pin(check):
    check()
