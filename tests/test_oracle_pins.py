"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from pins import PINS


@pytest.fixture(scope="module")
def ref():
    return oracle.default()


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(ref, name):
    PINS[name](ref)
