"""The CPU oracle against what the pages and mathematics fix (runs without a GPU)."""

import pytest

from oracle import kvq_oracle
from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(kvq_oracle)
