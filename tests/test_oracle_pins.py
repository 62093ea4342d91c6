"""The oracle against its pins (CPU only): hand-worked examples, closed forms,
torch's fp64 conv1d, invariants, SiLU and dtype conversions."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(ora, pin):
    pin(ora)
