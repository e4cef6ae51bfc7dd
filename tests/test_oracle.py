"""CPU checks of the oracle against facts fixed outside it (see oracle_pins.py, mask_pins.py)."""

import pytest

import mask_pins
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS + mask_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()


def test_flop_count():
    from oracle import attention_flops
    assert attention_flops(4, 16, 8192, 128, "none") == 4 * 4 * 16 * 8192 ** 2 * 128
    assert attention_flops(4, 16, 8192, 128, "causal") == 2 * 4 * 16 * 8192 ** 2 * 128
    assert attention_flops(1, 1, 128, 64, "bitmask") == 4 * 128 * 128 * 64
