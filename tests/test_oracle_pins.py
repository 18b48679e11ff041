"""The CPU oracle against its pins (closed forms, invariants, brute force, the
pages' worked numbers and a library special case).  No GPU needed."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)
