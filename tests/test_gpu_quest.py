"""Quest-style page-budget sparse decode on the GPU against the CPU oracle
(needs an MI355X): page summaries bit for bit, the page choice (exact wherever
the kept set is unique; where fp32 and fp64 scores order a near-tie
differently, both choices must be valid), and the end-to-end decode
(summaries, choice, per-head plan, run) against oracle.quest_attention."""

import numpy as np
import pytest
import torch

import oracle
from serving_attention_bsr_amd import lib
from serving_attention_bsr_amd import workloads as W
from tests.gpu_common import TOL, LSE_TOL, say

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


SUMMARY_CASES = [
    # name, kv_lens, h_kv, d, P, dtype
    ("bf16_p16", [17, 64, 300, 1], 8, 128, 16, "bf16"),
    ("bf16_p1_d64", [5, 40], 2, 64, 1, "bf16"),
    ("f32_p3_d256", [7, 100, 3], 2, 256, 3, "f32"),
]


@pytest.mark.parametrize("case", SUMMARY_CASES, ids=[c[0] for c in SUMMARY_CASES])
def test_page_summaries_are_exact(case):
    name, kv, h_kv, d, P, dtype = case
    say("summary", name)
    w = W.build(name, 71, [1] * len(kv), kv, P, h_kv, h_kv, d, dtype=dtype)  # NaN in unused slots
    k = w.k_pool.cuda()
    kmin, kmax = lib.page_summary(k, _dev(w.kv_indptr), _dev(w.kv_indices), _dev(w.last_page_len))
    torch.cuda.synchronize()
    emin, emax = oracle.page_summaries(w.k_pool.double().numpy(), w.kv_indptr, w.kv_indices, w.last_page_len, P)
    used = np.unique(w.kv_indices)
    got_min = kmin.double().cpu().numpy()[used]
    got_max = kmax.double().cpu().numpy()[used]
    assert np.array_equal(got_min, emin[used]) and np.array_equal(got_max, emax[used]), name


def _choose(w, budget):
    dev = torch.device("cuda:0")
    q, k = w.q.to(dev), w.k_pool.to(dev)
    kvp, kvi, last = _dev(w.kv_indptr), _dev(w.kv_indices), _dev(w.last_page_len)
    kmin, kmax = lib.page_summary(k, kvp, kvi, last)
    out_ptr = lib.quest_out_indptr(w.kv_indptr, w.num_kv_heads, budget)
    n_max = int(np.diff(w.kv_indptr).max())
    out = lib.quest_select(q, kmin, kmax, kvp, kvi, budget, _dev(out_ptr), n_max)
    torch.cuda.synchronize()
    return out_ptr, out.cpu().numpy()


def _check_choice(w, budget, out_ptr, got):
    """Returns the (request, KV head) pairs whose kept set equals the oracle's."""
    kmin, kmax = oracle.page_summaries(w.k_pool.double().numpy(), w.kv_indptr, w.kv_indices, w.last_page_len,
                                       w.page_size)
    sel = oracle.quest_selection(w.q.double().numpy(), kmin, kmax, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                 w.num_qo_heads, w.num_kv_heads, budget)
    same = set()
    differ = 0
    for r in range(w.batch):
        b, e = int(w.kv_indptr[r]), int(w.kv_indptr[r + 1])
        ids = np.asarray(w.kv_indices[b:e])
        sc = oracle.page_scores(w.q[r].double().numpy(), kmin[ids], kmax[ids], w.group)
        for hk in range(w.num_kv_heads):
            lo, hi = int(out_ptr[r * w.num_kv_heads + hk]), int(out_ptr[r * w.num_kv_heads + hk + 1])
            want = list(ids[sel[r][hk]])
            have = list(got[lo:hi])
            if have == want:
                same.add((r, hk))
                continue
            differ += 1
            # a near-tie at the cut: the last page is last, both lists are valid top sets
            assert len(have) == len(want) and have[-1] == want[-1], (r, hk)
            pos = {int(p): i for i, p in enumerate(ids)}
            hp = sorted(pos[int(p)] for p in have[:-1])
            assert [int(ids[i]) for i in hp] == have[:-1], "kept pages in logical order"
            cut = min(sc[hk, i] for i in sel[r][hk][:-1])
            for i in set(hp) ^ set(int(x) for x in sel[r][hk][:-1]):
                assert abs(sc[hk, i] - cut) <= 1e-5 * max(1.0, abs(cut)), (r, hk, i, sc[hk, i], cut)
    say("choice", dict(pairs=w.batch * w.num_kv_heads, differ_near_ties=differ))
    return same


CHOICE_CASES = [
    # name, kv_lens, h_qo, h_kv, d, P, dtype, budget
    ("mha_d128_b8", [900, 1000, 77, 16, 3000], 8, 8, 128, 16, "bf16", 8),
    ("gqa4_d64_b1", [100, 40, 17], 8, 2, 64, 4, "bf16", 1),
    ("gqa2_d256_all", [30, 100], 4, 2, 256, 16, "bf16", 64),
    ("f32_d128_b5", [500, 61], 4, 4, 128, 8, "f32", 5),
]


@pytest.mark.parametrize("case", CHOICE_CASES, ids=[c[0] for c in CHOICE_CASES])
def test_page_choice_matches_oracle(case):
    name, kv, h_qo, h_kv, d, P, dtype, budget = case
    say("choice", name)
    w = W.build(name, 72, [1] * len(kv), kv, P, h_qo, h_kv, d, dtype=dtype)
    out_ptr, got = _choose(w, budget)
    same = _check_choice(w, budget, out_ptr, got)
    assert len(same) >= 0.9 * w.batch * h_kv


def _quest_decode(w, budget, **kw):
    dev = torch.device("cuda:0")
    q, k, v = w.q.to(dev), w.k_pool.to(dev), w.v_pool.to(dev)
    out_ptr, got = _choose(w, budget)
    h = lib.BsrAttention(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, dtype=w.dtype,
                         logits_soft_cap=w.cap, max_batch=w.batch, max_total_qo=w.batch,
                         max_total_kv=max(int(w.kv_lens.max()), 1), device=0, **kw)
    info = h.plan_head_pages(w.qo_indptr, out_ptr, w.last_page_len)
    o, lse = h.run(q, k, v, _dev(got))
    torch.cuda.synchronize()
    h.check()
    return out_ptr, got, o.double().cpu().numpy(), lse.double().cpu().numpy(), info


QUEST_CASES = [
    # name, kv_lens, h_qo, h_kv, d, P, dtype, budget, cap
    ("long_mha_d128", [32768], 32, 32, 128, 16, "bf16", 64, 0.0),
    ("batch_gqa_d128_cap", [20000, 3000, 900, 64, 7000], 32, 8, 128, 16, "bf16", 32, 30.0),
    ("d64_p8_small", [400, 17, 1000], 8, 4, 64, 8, "bf16", 4, 0.0),
]


@pytest.mark.parametrize("case", QUEST_CASES, ids=[c[0] for c in QUEST_CASES])
def test_quest_decode_matches_oracle(case):
    name, kv, h_qo, h_kv, d, P, dtype, budget, cap = case
    say("quest", name)
    w = W.build(name, 73, [1] * len(kv), kv, P, h_qo, h_kv, d, dtype=dtype, cap=cap)
    out_ptr, got, o, lse, info = _quest_decode(w, budget)
    say("plan", info)
    same = _check_choice(w, budget, out_ptr, got)
    ro, rl, _ = oracle.quest_attention(w.q.double().numpy(), w.k_pool.double().numpy(), w.v_pool.double().numpy(),
                                       w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, P, h_qo, h_kv,
                                       w.scale, budget, cap=cap)
    atol, rtol = TOL[dtype]
    g = h_qo // h_kv
    checked = 0
    for (r, hk) in same:
        rows = slice(hk * g, hk * g + g)
        err = np.abs(o[r, rows] - ro[r, rows])
        assert np.all(err <= atol + rtol * np.abs(ro[r, rows])), (name, r, hk, float(err.max()))
        assert np.all(np.abs(lse[r, rows] - rl[r, rows]) <= LSE_TOL), (name, r, hk)
        checked += 1
    say("checked pairs", checked, "of", w.batch * h_kv)
    assert checked >= 0.9 * w.batch * h_kv
