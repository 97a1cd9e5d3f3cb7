"""GPU parity of the sliding-window mask against the oracle, with bitwise repeat
and graph replay after a re-plan.

The window is one of the mask variants of the FlashInfer explainer page
(Background, and paper section 3.2.3's LogitsMask functor); a query token sees
the W keys ending at its bottom-right aligned position.  Cases cover every body
that masks: the VALU decode body (bf16, fp32, FP8 K/V, soft-cap, chunks split by
a small grid), the 32-row MFMA body (one-key and 16-key pages), the 16-row D=256
MFMA body, a window of one key, non-causal windows and a window longer than the
KV.  The planner starts each tile at its window, so these runs also check that
the shortened chunks and their merges line up with the oracle.
"""

import pytest

from serving_attention_bsr_amd import workloads as W
from tests.gpu_common import compare, oracle_of, run_gpu, say

CASES = [
    # name, qo_lens, kv_lens, h_qo, h_kv, d, P, dtype, causal, cap, nwg, window
    ("win_decode_bf16_split", [1] * 6, [4000, 700, 64, 1, 300, 129], 32, 8, 128, 16, "bf16", False, 0.0, 16, 300),
    ("win_spec_f32", [2, 3, 1], [90, 333, 500], 8, 2, 64, 5, "f32", True, 0.0, 0, 37),
    ("win_decode_cap_d256", [1, 1, 1], [1000, 70, 2000], 16, 4, 256, 16, "bf16", False, 20.0, 0, 129),
    ("win_fp8_decode", [1] * 4, [3000, 100, 700, 1], 32, 8, 128, 16, "bf16_kv_fp8", True, 0.0, 0, 256),
    ("win_mfma_d128_causal_p1", [300, 33, 128], [700, 33, 1000], 32, 8, 128, 1, "bf16", True, 0.0, 8, 100),
    ("win_mfma_d128_p16", [200, 64], [2000, 64], 32, 8, 128, 16, "bf16", True, 0.0, 0, 513),
    ("win_mfma_d64_noncausal", [129, 64], [65, 300], 4, 4, 64, 16, "bf16", False, 0.0, 0, 40),
    ("win_mfma_d256_causal_split", [90, 17], [600, 17], 16, 4, 256, 1, "bf16", True, 0.0, 8, 77),
    ("win_one_mfma", [70, 5], [70, 80], 8, 2, 128, 3, "bf16", True, 0.0, 0, 1),
    ("win_longer_than_kv", [40, 1], [100, 64], 8, 2, 128, 16, "bf16", True, 0.0, 0, 5000),
    # the largest window with more queries than keys (non-causal)
    ("win_huge_noncausal", [129, 1], [65, 70], 8, 2, 128, 16, "bf16", False, 0.0, 0, 2**31 - 1),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_window_matches_oracle(case):
    name, qo, kv, h_qo, h_kv, d, P, dtype, causal, cap, nwg, window = case
    say("case", name)
    w = W.build(name, 31, qo, kv, P, h_qo, h_kv, d, dtype=dtype, causal=causal, cap=cap, window=window)
    o, lse, info = run_gpu(w, num_workgroups=nwg)
    say("plan", info)
    ro, rl = oracle_of(w)
    compare(w, o, lse, ro, rl, name)


@pytest.mark.gpu
def test_window_repeat_runs_are_bitwise_identical():
    """A windowed plan with split chunks and merges gives the same bits on every run."""
    import torch

    from tests.gpu_common import handle_for, to_gpu

    say("case window_repeat")
    w = W.named("batch_decode_window", batch=16, lo=100, hi=6000, window=1000)
    h = handle_for(w)
    q, k, v, idx = to_gpu(w)
    info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    assert info["num_partial_items"] > 0, "the case must exercise the merge"
    o0, l0 = h.run(q, k, v, idx)
    o0, l0 = o0.clone(), l0.clone()
    for _ in range(5):
        o, l = h.run(q, k, v, idx)
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16))
        assert torch.equal(l.view(torch.int32), l0.view(torch.int32))
    h.check()
    ro, rl = oracle_of(w)
    compare(w, o0.double().cpu().numpy(), l0.double().cpu().numpy(), ro, rl, "window_repeat")


@pytest.mark.gpu
def test_window_graph_replays_after_replan():
    """A captured windowed run() replays the current plan: re-plan new lengths and
    replay again; every replay matches the oracle."""
    import numpy as np
    import torch

    from tests.gpu_common import handle_for

    say("case window_graph")
    w1 = W.named("batch_decode_window", seed=41, batch=24, lo=64, hi=4000, window=700)
    w2 = W.named("batch_decode_window", seed=42, batch=24, lo=64, hi=4000, window=700)
    dev = torch.device("cuda:0")
    n_pages = max(w1.k_pool.shape[0], w2.k_pool.shape[0])
    n_idx = max(len(w1.kv_indices), len(w2.kv_indices))
    q = torch.empty(w1.q.shape, dtype=w1.q.dtype, device=dev)
    k = torch.empty((n_pages,) + tuple(w1.k_pool.shape[1:]), dtype=w1.k_pool.dtype, device=dev)
    v = torch.empty_like(k)
    idx = torch.zeros(n_idx, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=dev)
    h = handle_for(w1, max_total_kv=int(max(w1.kv_lens.sum(), w2.kv_lens.sum())))

    def load(w):
        q.copy_(w.q)
        k[: w.k_pool.shape[0]].copy_(w.k_pool)
        v[: w.v_pool.shape[0]].copy_(w.v_pool)
        idx[: len(w.kv_indices)].copy_(torch.from_numpy(np.ascontiguousarray(w.kv_indices)))
        h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
        torch.cuda.synchronize()

    load(w1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        h.run(q, k, v, idx, o, lse)  # warm the launch path outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        h.run(q, k, v, idx, o, lse)
    for w, label in ((w1, "first plan"), (w2, "re-plan")):
        if w is w2:
            load(w2)
        ro, rl = oracle_of(w)
        for rep in range(2):
            o.zero_()
            g.replay()
            torch.cuda.synchronize()
            compare(w, o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, f"{label} replay {rep}")
    h.check()
