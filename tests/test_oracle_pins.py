"""The oracle against its pins (CPU only)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check, oracle_lib):
    check(oracle_lib)
