"""The Quest-style page-budget oracle against its pins, and planted mistakes."""

import os
import types

import pytest

from oracle import quest as quest_oracle
from tests import quest_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "quest.py")

MUTANTS = {
    "score_max_side_only": ("np.maximum(qh * kmin_pages[:, hk, :], qh * kmax_pages[:, hk, :])",
                            "qh * kmax_pages[:, hk, :]"),
    "score_min_max_swapped_sign": ("np.maximum(qh * kmin_pages[:, hk, :], qh * kmax_pages[:, hk, :])",
                                   "np.minimum(qh * kmin_pages[:, hk, :], qh * kmax_pages[:, hk, :])"),
    "summary_counts_unused_slots": ("valid = page_size if i < e - 1 else int(last_page_len[r])\n            keys",
                                    "valid = page_size\n            keys"),
    "group_mean": ("out[hk] = np.maximum(out[hk], ub)", "out[hk] = out[hk] + ub / group if np.isfinite(out[hk]).all() else ub / group"),
    "last_page_not_forced": ("others = sorted(range(n - 1),", "others = sorted(range(n),"),
    "ties_to_later_page": ("key=lambda i: (-float(scores[i]), i)", "key=lambda i: (-float(scores[i]), -i)"),
    "lowest_scores_kept": ("key=lambda i: (-float(scores[i]), i)", "key=lambda i: (float(scores[i]), i)"),
    "budget_off_by_one": ("[: budget - 1]", "[:budget]"),
    "last_page_full": ("valid = page_size if b + pos < e - 1 else int(last_page_len[r])",
                       "valid = page_size"),
}


@pytest.mark.parametrize("pin", quest_pins.ALL_QUEST_PINS, ids=lambda p: p.__name__)
def test_quest_pin(pin):
    pin(quest_oracle)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_quest_pin_catches_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    src = src.replace(old, new).replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType(f"quest_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    caught = []
    for pin in quest_pins.ALL_QUEST_PINS:
        try:
            pin(mod)
        except Exception as exc:
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin detects mutant {name}"
