"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(None)
