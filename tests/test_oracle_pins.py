"""The oracle against what the pages and mathematics fix (see tests/oracle_pins.py)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()


def test_f16_conversion_against_f16c_exhaustive():
    """Every binary32 in [2^-25, 2^16] (both signs) and the edges outside it."""
    pins.check_f16_conversion_f16c(full=True)
