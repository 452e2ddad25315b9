"""The fp64 oracle against its pins (see pins.py for what each pin states)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    # small cases: one thread each (the suite runs in parallel workers)
    pin(oracle.Oracle(oracle.load().path, threads=1))
