"""The CPU oracle against facts fixed by the mathematics (closed forms, brute force,
a second formulation, hand-worked values and invariants).  CPU only."""
import pytest

import oracle
from oracle_pins import all_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load_library()


@pytest.mark.parametrize("name,pin", all_pins(), ids=[n for n, _ in all_pins()])
def test_pin(lib, name, pin):
    pin(lib)
