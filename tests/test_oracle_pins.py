"""The fp64 oracle against closed forms, invariants, brute force, library
routines and the pages' printed sizes (CPU only)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()
