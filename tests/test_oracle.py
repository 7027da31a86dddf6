"""CPU pins of the fp64 oracle (see oracle_pins.py for what each one fixes)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
