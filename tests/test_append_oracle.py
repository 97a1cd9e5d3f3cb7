"""The K/V append oracle against its pins, and planted mistakes that a pin must catch."""

import os
import types

import pytest

from oracle import append as append_oracle
from tests import append_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "append.py")

MUTANTS = {
    "positions_from_the_front": ("tau = int(l_kv[r]) - n_r + j", "tau = j"),
    "page_and_slot_swapped": ("kv_indices[kv_indptr[r] + tau // page_size]", "kv_indices[kv_indptr[r] + tau % page_size]"),
    "slot_off_by_one": ("slot[append_indptr[r] + j] = tau % page_size", "slot[append_indptr[r] + j] = (tau + 1) % page_size"),
    "overflow_wraps": ("            if tau < 0:\n                continue\n", ""),
    "v_gets_k": ("v_out[page[i], :, slot[i], :] = v_new[i]", "v_out[page[i], :, slot[i], :] = k_new[i]"),
    "pool_written_in_place": ("k_out = np.array(k_pool, copy=True)", "k_out = k_pool"),
}


@pytest.mark.parametrize("pin", append_pins.ALL_APPEND_PINS, ids=lambda p: p.__name__)
def test_append_pin(pin):
    pin(append_oracle)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_append_pin_catches_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"pattern for {name} must occur exactly once"
    src = src.replace(old, new).replace("from .attention import kv_lengths", "from oracle.attention import kv_lengths")
    mod = types.ModuleType(f"append_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    caught = []
    for pin in append_pins.ALL_APPEND_PINS:
        try:
            pin(mod)
        except Exception as exc:  # AssertionError, or a crash caused by the mistake
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin detects mutant {name}"
