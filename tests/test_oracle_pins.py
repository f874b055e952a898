"""The fp64 oracle against facts the mathematics fixes (no GPU)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.SEQUENTIAL_PINS, ids=lambda p: p.__name__)
def test_sequential_pin(pin):
    assert pin() < pins.TOL


def test_chunked_matches_bruteforce():
    assert pins.pin_bruteforce(chunk=16) < pins.TOL
    assert pins.pin_bruteforce(chunk=64) < pins.TOL


def test_chunked_matches_sequential():
    assert pins.pin_chunked_vs_sequential() < pins.TOL
