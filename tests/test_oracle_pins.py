"""The CPU oracle against its pins (closed forms, invariants, brute force,
library routines and the statistics printed on the pages)."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
