"""The CPU oracle against its pins (CPU only)."""
import pytest

from oracle import lora_oracle
from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(lora_oracle)
