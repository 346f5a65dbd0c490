"""The fp64 oracle against its pins (library routines, closed forms, invariants, brute force)."""
import pytest

from oracle import attn_oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def oracle():
    return attn_oracle.get()


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(oracle, check):
    check(oracle)
