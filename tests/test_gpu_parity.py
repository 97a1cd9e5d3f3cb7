"""HIP path against the CPU oracle, element by element (needs an MI355X)."""

import numpy as np
import pytest
import torch

from serving_attention_bsr_amd import lib
from serving_attention_bsr_amd import workloads as W
from tests.gpu_common import compare, handle_for, oracle_of, run_gpu, say, to_gpu

pytestmark = pytest.mark.gpu


SWEEP = [
    # name, qo_lens, kv_lens, h_qo, h_kv, d, P, dtype, causal, cap, nwg
    ("f32_d64_p16", [1, 1, 1, 1], [17, 64, 100, 255], 8, 2, 64, 16, "f32", False, 0.0, 0),
    ("f32_d64_split", [1, 1, 1, 1], [17, 64, 100, 255], 8, 2, 64, 16, "f32", False, 0.0, 64),
    ("f32_d128_p3_cap", [1, 1, 1], [1, 77, 1000], 8, 4, 128, 3, "f32", False, 10.0, 0),
    ("f32_d256_g1", [1, 1], [33, 500], 2, 2, 256, 16, "f32", False, 0.0, 0),
    ("bf16_d128_p16", [1] * 9, [1, 2, 31, 32, 33, 511, 512, 513, 3000], 32, 8, 128, 16, "bf16", False, 0.0, 0),
    ("bf16_d128_p1", [1] * 5, [7, 64, 129, 700, 2048], 32, 8, 128, 1, "bf16", False, 0.0, 0),
    ("bf16_d128_p5_split", [1] * 5, [7, 64, 129, 700, 2048], 32, 8, 128, 5, "bf16", False, 0.0, 16),
    ("bf16_d64_g8_rows8", [1, 1, 1], [100, 1000, 5], 16, 2, 64, 16, "bf16", False, 0.0, 0),
    ("bf16_d256_g4_cap", [1] * 4, [64, 300, 512, 1500], 16, 4, 256, 16, "bf16", False, 30.0, 0),
    ("bf16_d256_g2", [1] * 3, [10, 300, 900], 8, 4, 256, 7, "bf16", False, 0.0, 8),
    ("bf16_spec2_causal", [2, 2, 2], [2, 90, 333], 8, 2, 128, 16, "bf16", True, 0.0, 0),
    ("bf16_empty_rows", [1, 1, 1], [0, 40, 0], 8, 2, 128, 16, "bf16", False, 0.0, 0),
    ("bf16_g1_cap_split", [1] * 4, [4000, 1, 63, 65], 4, 4, 128, 16, "bf16", False, 5.0, 4),
    # MFMA tile body: wide folded rows (prefill), ragged tiles, causal diagonals
    ("mfma_d128_causal_p1", [40, 7, 70], [100, 7, 200], 32, 8, 128, 1, "bf16", True, 0.0, 0),
    ("mfma_d128_causal_p3_split", [300, 33], [700, 33], 32, 8, 128, 3, "bf16", True, 0.0, 8),
    ("mfma_d64_g1_nocausal", [129, 64], [65, 300], 4, 4, 64, 16, "bf16", False, 0.0, 0),
    ("mfma_d256_g4_cap", [50, 3], [400, 1000], 16, 4, 256, 16, "bf16", False, 20.0, 0),
    # D = 256 runs the 16-row body: causal, several 64-row tiles, a split chunk
    ("mfma_d256_causal_p1_split", [90, 17], [600, 17], 16, 4, 256, 1, "bf16", True, 0.0, 8),
    ("mfma_d128_g8_causal", [33, 200], [40, 200], 16, 2, 128, 2, "bf16", True, 0.0, 0),
    ("mixed_decode_prefill", [1, 50, 1, 3], [500, 120, 77, 3], 32, 8, 128, 4, "bf16", True, 0.0, 16),
    ("mfma_empty_kv_rows", [20, 5], [0, 9], 8, 2, 128, 16, "bf16", False, 0.0, 0),
    # LDS-direct gather: one-key pages at D = 64, odd page sizes at D = 256, many tiles
    ("mfma_d64_causal_p1", [70, 130], [200, 130], 8, 2, 64, 1, "bf16", True, 0.0, 0),
    ("mfma_d256_p5_split", [70, 20], [333, 800], 8, 2, 256, 5, "bf16", False, 0.0, 8),
    ("mfma_d128_p16_long", [100, 64], [3000, 64], 8, 2, 128, 16, "bf16", True, 0.0, 0),
    # one-key-page instances with the soft-cap (odd and even tile counts)
    ("mfma_d128_p1_cap", [60, 200], [60, 900], 16, 4, 128, 1, "bf16", False, 30.0, 0),
    ("mfma_d256_p1_cap_split", [70, 9], [500, 9], 8, 2, 256, 1, "bf16", True, 15.0, 8),
]


@pytest.mark.parametrize("case", SWEEP, ids=[c[0] for c in SWEEP])
def test_sweep(case):
    name, qo, kv, h_qo, h_kv, d, P, dtype, causal, cap, nwg = case
    say("case", name)
    w = W.build(name, 21, qo, kv, P, h_qo, h_kv, d, dtype=dtype, causal=causal, cap=cap)
    o, lse, info = run_gpu(w, num_workgroups=nwg)
    say("plan", info)
    ro, rl = oracle_of(w)
    compare(w, o, lse, ro, rl, name)


# 64-row tiles at head dim 128 (rows of at most 64 folded rows on average): every
# instance of the short-tile kernel (soft-cap, one key per page), ragged tiles,
# causal diagonals, split chunks, decode-sized rows among them
SHORT = [
    ("short_d128_causal_p16", [3, 5, 8, 16, 12, 2], [100, 3000, 64, 900, 17, 2], 32, 8, 128, 16, False, 0.0, 0),
    ("short_d128_g2_p3_split", [20, 31, 5], [700, 31, 2000], 8, 4, 128, 3, True, 0.0, 16),
    ("short_d128_g8_cap", [8, 3, 6], [1500, 40, 333], 16, 2, 128, 16, False, 25.0, 0),
    ("short_d128_p1_causal", [16, 9, 4], [2048, 9, 130], 32, 8, 128, 1, True, 0.0, 8),
    ("short_d128_p1_cap", [11, 16], [90, 4000], 16, 4, 128, 1, True, 30.0, 0),
]


@pytest.mark.parametrize("case", SHORT, ids=[c[0] for c in SHORT])
def test_short_tiles(case):
    name, qo, kv, h_qo, h_kv, d, P, causal, cap, nwg = case
    say("case", name)
    w = W.build(name, 23, qo, kv, P, h_qo, h_kv, d, dtype="bf16", causal=causal, cap=cap)
    o, lse, info = run_gpu(w, num_workgroups=nwg)
    say("plan", info)
    assert info["q_tile"] == 64 and info["kernel"] == 2
    ro, rl = oracle_of(w)
    compare(w, o, lse, ro, rl, name)


@pytest.mark.parametrize("name", ["tiny_decode_f32", "batch_decode", "skewed_long_decode", "batch_decode_window"])
def test_named_decode(name):
    say("workload", name)
    w = W.named(name)
    o, lse, info = run_gpu(w)
    say("plan", info)
    ro, rl = oracle_of(w)
    compare(w, o, lse, ro, rl, name)


def test_named_prefill():
    say("workload ragged_causal_prefill")
    w = W.named("ragged_causal_prefill")
    o, lse, info = run_gpu(w)
    ro, rl = oracle_of(w)
    compare(w, o, lse, ro, rl, "ragged_causal_prefill")


def test_named_composable():
    say("workload shared_prefix_composable")
    w = W.named("shared_prefix_composable")
    o, lse, info = run_gpu(w, composable=True)
    ro, rl = oracle_of(w, composable=True)
    compare(w, o, lse, ro, rl, "shared_prefix_composable")


def test_repeat_runs_are_bitwise_identical():
    w = W.named("skewed_long_decode", long_len=16384, n_short=7)
    h = handle_for(w)
    q, k, v, idx = to_gpu(w)
    info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    assert info["num_partial_items"] > 0, "the case must exercise the merge"
    o0, l0 = h.run(q, k, v, idx)
    o0, l0 = o0.clone(), l0.clone()
    for _ in range(10):
        o, l = h.run(q, k, v, idx)
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16))
        assert torch.equal(l.view(torch.int32), l0.view(torch.int32))
    h.check()


def test_physical_page_permutation_keeps_bits():
    w = W.named("batch_decode", batch=16, lo=100, hi=3000)
    o, lse, _ = run_gpu(w)
    rng = np.random.default_rng(5)
    perm = rng.permutation(w.k_pool.shape[0])  # new position of each page
    inv = np.argsort(perm)
    w2 = W.named("batch_decode", batch=16, lo=100, hi=3000)
    w2.k_pool = w.k_pool[torch.from_numpy(inv)]
    w2.v_pool = w.v_pool[torch.from_numpy(inv)]
    w2.kv_indices = perm[w.kv_indices].astype(np.int32)
    o2, lse2, _ = run_gpu(w2)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_graph_capture_replays_after_replan():
    """A captured run() replays the current plan: re-plan new lengths, replay again."""
    w1 = W.named("batch_decode", seed=31, batch=24, lo=64, hi=4000)
    w2 = W.named("batch_decode", seed=32, batch=24, lo=64, hi=4000)
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
    eager_o, eager_l = o.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        h.run(q, k, v, idx, o, lse)
    ro, rl = oracle_of(w1)
    for rep in range(3):
        o.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), eager_o.view(torch.int16)), f"replay {rep} differs from eager"
        compare(w1, o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, f"graph replay {rep}")
    load(w2)
    ro2, rl2 = oracle_of(w2)
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        compare(w2, o.double().cpu().numpy(), lse.double().cpu().numpy(), ro2, rl2, f"replan replay {rep}")
    h.check()


def test_merge_states_matches_oracle():
    import oracle

    rng = np.random.default_rng(3)
    rows, d = 1000, 128
    oa = rng.standard_normal((rows, d)).astype(np.float32)
    ob = rng.standard_normal((rows, d)).astype(np.float32)
    la = (rng.standard_normal(rows) * 5).astype(np.float32)
    lb = (rng.standard_normal(rows) * 5).astype(np.float32)
    la[:10] = -np.inf
    lb[5:15] = -np.inf
    oa[:10] = 0
    ob[5:15] = 0
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(a).to(dev)
    o, l = lib.merge_states(t(oa), t(la), t(ob), t(lb))
    torch.cuda.synchronize()
    ro, rl = oracle.merge_state(oa, la, ob, lb)
    np.testing.assert_allclose(o.cpu().numpy(), ro, atol=2e-6, rtol=2e-6)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(l.cpu().numpy()))
    np.testing.assert_allclose(l.cpu().numpy()[fin], rl[fin], atol=2e-6, rtol=2e-6)
    # in place (output aliases the first input)
    oa_t, la_t = t(oa), t(la)
    lib.merge_states(oa_t, la_t, t(ob), t(lb), oa_t, la_t)
    torch.cuda.synchronize()
    np.testing.assert_allclose(oa_t.cpu().numpy(), ro, atol=2e-6, rtol=2e-6)


def test_two_per_cu_plan_is_balanced_in_time():
    """On a device handle the two-per-CU MFMA grid gives each CU's second workgroup
    (ids #CU .. 2 #CU - 1) about 11/16 of the first one's load, and every work item
    is queued exactly once."""
    from tests import plan_blob

    w = W.named("ragged_causal_prefill", tensors=False)
    h = lib.BsrAttention(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, dtype=w.dtype, causal=w.causal,
                         max_batch=w.batch, max_total_qo=int(w.qo_indptr[-1]), max_total_kv=int(w.kv_lens.sum()),
                         device=0, static_queues=True)
    info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say("plan", info, "cus", cus)
    assert info["kernel"] == 2 and info["num_workgroups"] == 2 * cus
    plan = plan_blob.decode(h.plan_bytes())
    ptr, items = plan["item_ptr"], plan["items"]
    assert ptr[-1] == len(items) == info["num_items"]
    keys = items["kv_end"] - items["kv_begin"]
    load = np.array([keys[ptr[i]:ptr[i + 1]].sum() for i in range(2 * cus)], dtype=np.float64)
    ratio = load[cus:].mean() / load[:cus].mean()
    say("second / first slot load", ratio)
    assert 0.6 < ratio < 0.78, ratio
    # every (row block, head, query tile) unit appears once: no duplicated item
    sig = set(zip(items["qo_begin"].tolist(), items["kv_head"].tolist(), items["kv_begin"].tolist()))
    assert len(sig) == len(items)
