"""The oracle against its pins (closed forms, brute force, worked examples,
library routines, invariants); see tests/oracle_pins.py."""
import pytest

import oracle.s2o as S2O
from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(S2O)
