"""The E4M3 decoder of the oracle against its pins, and planted mistakes."""

import os
import types

import pytest

from oracle import fp8 as fp8_oracle
from tests import fp8_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "fp8.py")

MUTANTS = {
    "bias_8": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "subnormal_scale": ("m * 2.0 ** -9", "m * 2.0 ** -10"),
    "no_nan": ("return np.where((e == 15) & (m == 7), np.nan, value)", "return value"),
    "mantissa_over_16": ("(1.0 + m / 8.0)", "(1.0 + m / 16.0)"),
}


@pytest.mark.parametrize("pin", fp8_pins.ALL_FP8_PINS, ids=lambda p: p.__name__)
def test_fp8_pin(pin):
    pin(fp8_oracle)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_fp8_pin_catches_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"fp8_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    caught = []
    for pin in fp8_pins.ALL_FP8_PINS:
        try:
            pin(mod)
        except Exception as exc:
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin detects mutant {name}"
