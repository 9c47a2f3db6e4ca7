"""The CPU oracle against its pins (exact rational brute force, integer-exact
cases, closed forms and the invariants the pages state)."""

import pytest

import oracle.ref as ref
from tests.oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(ref)
