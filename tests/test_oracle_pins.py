"""The CPU oracle against its pins (see oracle_pins.py for what each rests on)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
