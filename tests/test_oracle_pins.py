"""The oracle against brute force, a library routine, closed forms and invariances."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    problems = pin()
    assert problems == [], problems
