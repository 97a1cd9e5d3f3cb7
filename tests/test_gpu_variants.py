"""ALiBi and tree masks (the variant functors of the FlashInfer explainer page's
Background and paper section 3.2.3; tree masks for speculative decoding, Quick
read item 1) on every attention body, against the CPU oracle (needs an MI355X).

Bodies: the decode body at 4 and 8 folded rows (bf16, fp32, FP8 K/V), the 32-row
MFMA body (head dim 64 and 128, one-key and 16-key pages), the 16-row MFMA body
(head dim 256), and the mixed grid; split plans exercise the merge; a windowed
case combines all masks; a repeat checks the bits.
"""

import numpy as np
import pytest
import torch

from serving_attention_bsr_amd import lib
from serving_attention_bsr_amd import workloads as W
from tests.gpu_common import compare, handle_for, oracle_of, say, to_gpu
from tests.variant_pins import random_tree

pytestmark = pytest.mark.gpu


def alibi_slopes(h_qo):
    """The ALiBi paper's geometric slopes 2^(-8 (h + 1) / H)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / h_qo) for h in range(h_qo)])


CASES = [
    # name, qo_lens, kv_lens, h_qo, h_kv, d, P, dtype, causal, cap, window, nwg, alibi, tree
    ("decode4_alibi_split", [1] * 5, [7, 64, 700, 3000, 129], 32, 8, 128, 16, "bf16", False, 0.0, 0, 16, True, False),
    ("decode4_alibi_cap", [1] * 4, [64, 300, 512, 1500], 16, 4, 256, 16, "bf16", False, 30.0, 0, 0, True, False),
    ("decode8_tree_causal", [2, 2, 1, 2], [90, 2000, 40, 2], 32, 8, 128, 16, "bf16", True, 0.0, 0, 16, False, True),
    ("decode8_tree_alibi_g2", [4, 3, 1], [500, 37, 64], 8, 4, 64, 5, "bf16", True, 0.0, 0, 8, True, True),
    ("f32_alibi_tree", [2, 1, 1, 2], [17, 64, 100, 255], 8, 4, 64, 16, "f32", True, 0.0, 0, 16, True, True),
    ("fp8_alibi_tree", [2, 1, 2], [300, 1200, 64], 32, 8, 128, 16, "bf16_kv_fp8", True, 0.0, 0, 16, True, True),
    ("mfma128_p1_alibi_causal", [300, 77], [700, 77], 32, 8, 128, 1, "bf16", True, 0.0, 0, 0, True, False),
    ("mfma128_tree_split", [16, 64, 33], [2000, 900, 33], 32, 8, 128, 16, "bf16", True, 0.0, 0, 16, False, True),
    ("mfma128_tree_alibi_cap", [40, 9], [400, 60], 16, 4, 128, 3, "bf16", True, 20.0, 0, 0, True, True),
    ("mfma64_alibi_noncausal", [129, 64], [65, 300], 4, 4, 64, 16, "bf16", False, 0.0, 0, 0, True, False),
    ("mfma256_alibi_tree_split", [48, 17], [600, 500], 16, 4, 256, 1, "bf16", True, 0.0, 0, 8, True, True),
    ("mixed_alibi_tree", [1, 50, 2, 3], [500, 120, 77, 3], 32, 8, 128, 4, "bf16", True, 0.0, 0, 16, True, True),
    ("window_alibi_tree", [1, 30, 4], [3000, 900, 2000], 32, 8, 128, 16, "bf16", True, 0.0, 700, 16, True, True),
]


def _run(case, repeat=0):
    name, qo, kv, h_qo, h_kv, d, P, dtype, causal, cap, window, nwg, use_alibi, use_tree = case
    say("case", name)
    w = W.build(name, 61, qo, kv, P, h_qo, h_kv, d, dtype=dtype, causal=causal, cap=cap, window=window)
    rng = np.random.default_rng(62)
    slopes = alibi_slopes(h_qo) if use_alibi else None
    trees = [random_tree(rng, n) for n in qo] if use_tree else None
    h = handle_for(w, num_workgroups=nwg, alibi_slopes=slopes)
    q, k, v, idx = to_gpu(w)
    if use_tree:
        info = h.plan_tree_mask(w.qo_indptr, w.kv_indptr, w.last_page_len, trees)
    else:
        info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    say("plan", info)
    o, lse = h.run(q, k, v, idx)
    torch.cuda.synchronize()
    h.check()
    for rep in range(repeat):
        o2, l2 = h.run(q, k, v, idx)
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int16) if o2.dtype == torch.bfloat16 else o2.view(torch.int32),
                           o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32)), rep
        assert torch.equal(l2.view(torch.int32), lse.view(torch.int32)), rep
    ro, rl = oracle_of(w, alibi_slopes=slopes, tree_masks=trees)
    compare(w, o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, name)
    return info


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_variant_case(case):
    _run(case)


def test_variant_split_plan_repeats_bitwise():
    info = _run(("repeat_tree_alibi", [2, 2, 48], [9000, 300, 4000], 32, 8, 128, 16, "bf16", True, 0.0, 0, 32, True,
                 True), repeat=5)
    assert info["num_partial_items"] > 0


def test_named_spec_decode_tree():
    """The tree-masked speculative-decoding workload the benchmark times, in full."""
    say("workload spec_decode_tree")
    w = W.named("spec_decode_tree")
    trees = W.draft_trees(w.qo_lens, 10)
    h = handle_for(w)
    q, k, v, idx = to_gpu(w)
    info = h.plan_tree_mask(w.qo_indptr, w.kv_indptr, w.last_page_len, trees)
    say("plan", info)
    o, lse = h.run(q, k, v, idx)
    torch.cuda.synchronize()
    h.check()
    ro, rl = oracle_of(w, tree_masks=trees)
    compare(w, o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, "spec_decode_tree")
