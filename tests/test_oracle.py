"""The fp64 CPU oracles (RMSNorm, LayerNorm) against their pins (CPU only)."""
import pytest

import oracle
from oracle import layernorm_oracle
from tests import oracle_pins, oracle_pins_ln


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


@pytest.mark.parametrize("pin", oracle_pins_ln.ALL_PINS, ids=lambda p: p.__name__)
def test_layernorm_oracle_pin(pin):
    pin(layernorm_oracle)
