"""CPU pins of the fp64 oracle (see oracle_pins.py for what pins what)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL, ids=lambda f: f.__name__)
def test_pin(check):
    check()
