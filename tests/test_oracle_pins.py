"""The fp64 oracle against its pins (CPU only): fixtures worked by hand from the pages' equations,
closed forms, special cases, library routines in float64 and finite differences."""
import pytest

import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
