"""The oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=[p.__name__ for p in oracle_pins.PINS])
def test_pin(orc, pin):
    pin(orc)


def test_oracle_is_not_a_mutant(orc):
    assert orc.mutant == 0
