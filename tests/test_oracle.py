"""The fp64 CPU oracles (RMSNorm, LayerNorm, RoPE, SwiGLU) against their pins (CPU only)."""
import pytest

import oracle
from oracle import layernorm_oracle, rope_oracle, swiglu_oracle
from tests import oracle_pins, oracle_pins_ln, oracle_pins_rope, oracle_pins_swiglu


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)


@pytest.mark.parametrize("pin", oracle_pins_ln.ALL_PINS, ids=lambda p: p.__name__)
def test_layernorm_oracle_pin(pin):
    pin(layernorm_oracle)


@pytest.mark.parametrize("pin", oracle_pins_rope.ALL_PINS, ids=lambda p: p.__name__)
def test_rope_oracle_pin(pin):
    pin(rope_oracle)


@pytest.mark.parametrize("pin", oracle_pins_swiglu.ALL_PINS, ids=lambda p: p.__name__)
def test_swiglu_oracle_pin(pin):
    pin(swiglu_oracle)
