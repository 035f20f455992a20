"""The oracle against its pins (library routine, brute force, closed forms, invariants)."""

import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_battery_is_not_empty():
    assert len(P.ALL_PINS) >= 15
