"""The oracle's sliding-window mask against its pins, and planted mistakes."""

import os
import types

import pytest

from oracle import attention as att_oracle
from tests import window_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")

MUTANTS = {
    "window_off_by_one": ("np.arange(l_qo) - window + 1", "np.arange(l_qo) - window"),
    "strict_lower_bound": ("cols >= np.asarray(lowest)", "cols > np.asarray(lowest)"),
    "window_ignored": ("if window > 0:", "if window < 0:"),
    "window_from_front": ("lowest = l_kv - l_qo + np.arange(l_qo) - window + 1",
                          "lowest = np.arange(l_qo) - window + 1"),
}


@pytest.mark.parametrize("pin", window_pins.ALL_WINDOW_PINS, ids=lambda p: p.__name__)
def test_window_pin(pin):
    pin(att_oracle)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_window_pin_catches_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"window_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    caught = []
    for pin in window_pins.ALL_WINDOW_PINS:
        try:
            pin(mod)
        except Exception as exc:
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin detects mutant {name}"
