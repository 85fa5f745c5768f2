"""The oracle against its independent pins (closed forms, SciPy/LAPACK,
invariants the pages state, brute force).  CPU only."""
import pytest

import oracle.nystrom as o
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(o)
