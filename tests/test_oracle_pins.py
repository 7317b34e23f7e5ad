"""The naive fp64 oracle against the pages' worked examples, closed forms,
invariants and torch's float64 CPU attention."""

import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)
