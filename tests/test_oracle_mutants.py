"""Plant plausible mistakes in a copy of the oracle; at least one pin must catch each.

The copy is made from the oracle's source text with one substitution and executed
as a fresh module on the CPU; the real oracle is untouched.
"""

import math
import json
import os
import types

import pytest

from tests import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")

MUTANTS = {
    "page_slot_swapped": ("tau // page_size]", "tau % page_size]"),
    "last_page_len_ignored": ("l_kv = (n_pages - 1) * page_size + int(last_page_len[r])", "l_kv = n_pages * page_size"),
    "gqa_modulo_mapping": ("hk = h // g\n            bias = None", "hk = h % num_kv_heads\n            bias = None"),
    "scale_dropped": ("s = scale * (q @ k.T)", "s = (q @ k.T)"),
    "k_transposed_with_v": ("out[live] = (w @ v) / z[:, None]", "out[live] = (w @ k) / z[:, None]"),
    "cap_factor_dropped": ("s = cap * np.tanh(s / cap)", "s = np.tanh(s / cap)"),
    "cap_after_scale_twice": ("s = cap * np.tanh(s / cap)", "s = cap * np.tanh(scale * s / cap)"),
    "causal_top_left": ("visible = l_kv - l_qo + np.arange(l_qo)", "visible = np.arange(l_qo)"),
    "causal_off_by_one": ("s = np.where(cols <= np.asarray(visible)[:, None], s, -np.inf)", "s = np.where(cols < np.asarray(visible)[:, None], s, -np.inf)"),
    "lse_missing_max": ("lse[live] = m_live + np.log(z)", "lse[live] = np.log(z)"),
    "o_not_normalised": ("out[live] = (w @ v) / z[:, None]", "out[live] = (w @ v)"),
    "merge_wrong_weight_sign": ("w_b = np.where(np.isfinite(lse_b), np.exp(lse_b - m_safe), 0.0)", "w_b = np.where(np.isfinite(lse_b), np.exp(m_safe - lse_b), 0.0)"),
    "merge_reuses_a_weight": ("o = (w_a[..., None] * o_a + w_b[..., None] * o_b)", "o = (w_a[..., None] * o_a + w_a[..., None] * o_b)"),
    "merge_lse_no_log": ("lse = np.where(empty, -np.inf, m_safe + np.log(z_safe))", "lse = np.where(empty, -np.inf, m_safe + z_safe - 1.0)"),
    "composable_offset_dropped": ('kv_indptr = np.asarray(f["kv_indptr"], dtype=np.int64) + int(f["kv_indices_offset"])', 'kv_indptr = np.asarray(f["kv_indptr"], dtype=np.int64)'),
    "softmax_exponent_perturbed": ("w = np.exp(s_live - m_live[:, None])", "w = np.exp(s_live - m_live[:, None] + 1e-3 * s_live)"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"pattern for {name} must occur exactly once"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name):
    mod = _mutant(name)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as exc:  # AssertionError, or a crash caused by the mistake
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin detects mutant {name}"


def test_golden_values_match_their_derivations():
    """Each stored closed-form value is re-derived from its expression with math only."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    env = {"e": math.e, "exp": math.exp, "log": math.log, "tanh": math.tanh, "__builtins__": {}}
    for c in cases:
        der = c["derivation"]
        assert abs(eval(der["lse"], env) - c["lse"]) <= 1e-15
        assert abs(eval(der["o0"], env) - c["o"][0]) <= 1e-15
        assert abs(eval(der["o1"], env) - c["o"][1]) <= 1e-15
