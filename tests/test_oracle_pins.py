"""CPU pins of the oracle (no GPU)."""
import pytest

from tests import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
