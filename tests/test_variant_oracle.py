"""The oracle's ALiBi bias and tree masks against their pins, and planted mistakes."""

import json
import math
import os
import types

import pytest

from oracle import attention as att_oracle
from tests import variant_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")

MUTANTS = {
    "alibi_sign_flipped": ("(np.arange(l_kv)[None, :] - positions[:, None])",
                           "(positions[:, None] - np.arange(l_kv)[None, :])"),
    "alibi_top_left_positions": ("positions = l_kv - l_qo + np.arange(l_qo)", "positions = np.arange(l_qo)"),
    "alibi_position_off_by_one": ("positions = l_kv - l_qo + np.arange(l_qo)",
                                  "positions = l_kv - l_qo + 1 + np.arange(l_qo)"),
    "alibi_after_cap": ("    if bias is not None:\n        s = s + np.asarray(bias, dtype=np.float64)\n"
                        "    if cap > 0.0:\n        s = cap * np.tanh(s / cap)\n",
                        "    if cap > 0.0:\n        s = cap * np.tanh(s / cap)\n"
                        "    if bias is not None:\n        s = s + np.asarray(bias, dtype=np.float64)\n"),
    "alibi_slope_of_kv_head": ("float(alibi_slopes[h])", "float(alibi_slopes[hk])"),
    "alibi_scaled": ("s = s + np.asarray(bias, dtype=np.float64)", "s = s + scale * np.asarray(bias, dtype=np.float64)"),
    "tree_transposed": ("allowed[:, l_kv - l_qo :] = tree", "allowed[:, l_kv - l_qo :] = tree.T"),
    "tree_at_front": ("allowed[:, l_kv - l_qo :] = tree", "allowed[:, :l_qo] = tree"),
    "tree_hides_prefix": ("allowed = np.ones((l_qo, l_kv), dtype=bool)", "allowed = np.zeros((l_qo, l_kv), dtype=bool)"),
    "tree_ignored": ("s = np.where(np.asarray(allowed, dtype=bool), s, -np.inf)", "s = s"),
}


@pytest.mark.parametrize("pin", variant_pins.ALL_VARIANT_PINS, ids=lambda p: p.__name__)
def test_variant_pin(pin):
    pin(att_oracle)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_variant_pin_catches_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"variant_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    caught = []
    for pin in variant_pins.ALL_VARIANT_PINS:
        try:
            pin(mod)
        except Exception as exc:
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin detects mutant {name}"


def test_variant_golden_values_match_their_derivations():
    """Each stored closed-form value is re-derived from its expression with math only."""
    with open(variant_pins.GOLDEN) as f:
        cases = json.load(f)["cases"]
    env = {"exp": math.exp, "log": math.log, "tanh": math.tanh, "__builtins__": {}}
    for c in cases:
        der = c["derivation"]
        assert abs(eval(der["lse"], env) - c["lse"]) <= 1e-15
        assert abs(eval(der["o0"], env) - c["o"][0]) <= 1e-15
        assert abs(eval(der["o1"], env) - c["o"][1]) <= 1e-15
