"""The host planner, through a host-only handle of the real library (no GPU).

* A CPU float64 executor runs the decoded plan (work items, then the merge map)
  and must reproduce the oracle's result: every (query, key) pair is covered
  exactly once and every merge reads states that were written.
* Plan invariants from the pages (Core mechanism 6 and 7 of the FlashInfer
  explainer page, paper Algorithm 1 and Appendix D.2/D.3): chunks never exceed
  L_kv, only split work writes partial states, at most 2 * #workgroups partial
  chunks, longest-first queues, byte-identical plans for identical lengths.
* Validation errors are returned before anything is launched.
"""

import numpy as np
import pytest

import oracle
from serving_attention_bsr_amd import lib
from serving_attention_bsr_amd import workloads as W
from tests import plan_blob


def host_handle(h_qo, h_kv, d, P, dtype="bf16", causal=False, cap=0.0, nwg=8, **kw):
    args = dict(
        num_qo_heads=h_qo, num_kv_heads=h_kv, head_dim=d, page_size=P, dtype=dtype, causal=causal,
        logits_soft_cap=cap, num_workgroups=nwg, device=-1, max_batch=512, max_total_qo=1 << 16,
        max_total_kv=1 << 24,
    )
    args.update(kw)
    return lib.BsrAttention(**args)


def f64(t):
    return t.double().numpy()


CASES = [
    # name, qo_lens, kv_lens, h_qo, h_kv, d, P, dtype, causal, cap, nwg, min_chunk
    ("decode_split", [1, 1, 1, 1], [17, 64, 100, 255], 8, 2, 64, 16, "f32", False, 0.0, 16, 64),
    ("decode_one_wg", [1, 1, 1], [300, 5, 129], 8, 2, 64, 3, "f32", False, 0.0, 1, 64),
    ("decode_cap_many_wg", [1] * 6, [700, 64, 65, 1, 300, 129], 4, 4, 64, 16, "bf16", False, 5.0, 32, 64),
    ("spec_decode_rows8", [2, 2, 1], [200, 90, 333], 8, 2, 64, 5, "bf16", True, 0.0, 8, 64),
    ("prefill_causal_tiles", [40, 7, 70], [100, 7, 200], 8, 2, 64, 1, "bf16", True, 0.0, 8, 64),
    ("prefill_noncausal", [33, 1], [90, 450], 4, 1, 64, 2, "bf16", False, 2.0, 5, 64),
    ("mixed_decode_prefill", [1, 50, 1, 3], [500, 120, 77, 3], 8, 2, 64, 4, "bf16", True, 0.0, 12, 64),
    ("empty_rows", [1, 0, 1, 2], [0, 5, 70, 0], 4, 2, 64, 4, "bf16", False, 0.0, 4, 64),
    ("fp32_long_queries", [20, 3], [40, 300], 8, 2, 64, 16, "f32", True, 0.0, 8, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_plan_executes_to_oracle(case):
    name, qo, kv, h_qo, h_kv, d, P, dtype, causal, cap, nwg, min_chunk = case
    w = W.build(name, 7, qo, kv, P, h_qo, h_kv, d, dtype=dtype, causal=causal, cap=cap)
    h = host_handle(h_qo, h_kv, d, P, dtype, causal, cap, nwg, min_kv_chunk=min_chunk)
    info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    plan = plan_blob.decode(h.plan_bytes())
    assert plan["header"]["num_wg"] == nwg == info["num_workgroups"]
    q, k, v = f64(w.q), f64(w.k_pool), f64(w.v_pool)
    o, lse, written = plan_blob.execute(plan, q, k, v, w.kv_indices, w.group, P, w.scale, cap)
    ro, rl = oracle.bsr_attention(
        q, k, v, w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, P, h_qo, h_kv, w.scale, causal, cap
    )
    assert np.all(written == 1), "every (token, head) is written exactly once"
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], rl[fin], rtol=1e-12, atol=1e-12)


def test_plan_splits_and_merges_when_work_is_long():
    w = W.build("split", 3, [1, 1], [5000, 64], 16, 8, 2, 64, dtype="bf16", tensors=False)
    h = host_handle(8, 2, 64, 16, nwg=8)
    info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    assert info["num_partial_items"] > 0 and info["num_merge_tasks"] == 2
    plan = plan_blob.decode(h.plan_bytes())
    partial = plan["items"]["flags"] & plan_blob.ITEM_PARTIAL != 0
    # the short request is not split and writes directly (paper Appendix D.2)
    short = plan["items"][(plan["items"]["qo_begin"] == 1)]
    assert np.all(short["flags"] & plan_blob.ITEM_PARTIAL == 0)
    assert np.all(plan["items"]["kv_end"][partial] - plan["items"]["kv_begin"][partial] <= info["kv_chunk"])


@pytest.mark.parametrize("cost_mfma", [0, 16, 400])
def test_composable_plan_executes_to_oracle(cost_mfma):
    w = W.shared_prefix_composable(
        seed=9, branches=6, prefix_len=48, suf_lo=1, suf_hi=40, page_size=16, num_qo_heads=8, num_kv_heads=2,
        head_dim=64,
    )
    h = host_handle(8, 2, 64, 16, nwg=6, cost_mfma=cost_mfma)
    fm = [f.as_dict() for f in w.formats]
    info = h.plan_composable(fm, w.batch)
    assert info["kernel"] == lib.KERNEL_MIXED
    plan = plan_blob.decode(h.plan_bytes())
    q, k, v = f64(w.q), f64(w.k_pool), f64(w.v_pool)
    o, lse, written = plan_blob.execute(plan, q, k, v, w.kv_indices_formats, w.group, 16, w.scale, 0.0)
    ro, rl = oracle.composable_attention(q, k, v, fm, w.kv_indices_formats, 16, 8, 2, w.scale)
    assert np.all(written == 1)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


def test_mixed_grid_weights_mfma_tokens():
    """In a grid that runs both bodies, an MFMA unit's KV tokens cost cost_mfma/16
    decode tokens: a heavier weight cuts the shared prefix into more, shorter
    pieces, and at the default the prefix work is spread over every workgroup
    (each holds the same number of MFMA pieces, give or take one).  Plans with one
    body do not depend on the weight."""
    w = W.shared_prefix_composable(tensors=False)
    fm = [f.as_dict() for f in w.formats]
    mb = w.batch + sum(len(f.qo_indptr) - 1 for f in w.formats)

    def plan(cost_mfma):
        h = host_handle(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, nwg=256, max_batch=mb,
                        cost_mfma=cost_mfma, static_queues=True)
        info = h.plan_composable(fm, w.batch)
        return info, plan_blob.decode(h.plan_bytes())

    light_info, light = plan(16)
    heavy_info, heavy = plan(0)
    mf = lambda p: p["items"][(p["items"]["flags"] & plan_blob.ITEM_MFMA) != 0]
    assert len(mf(heavy)) > len(mf(light))
    lens = lambda p: mf(p)["kv_end"] - mf(p)["kv_begin"]
    assert lens(heavy).max() < lens(light).max()
    ptr = heavy["item_ptr"]
    nwg = heavy["header"]["num_wg"]
    per_wg = [int(((heavy["items"][ptr[i]:ptr[i + 1]]["flags"] & plan_blob.ITEM_MFMA) != 0).sum()) for i in range(nwg)]
    assert len(mf(heavy)) >= nwg
    assert max(per_wg) - min(per_wg) <= 1
    d = W.batch_decode(tensors=False)
    bytes_for = []
    for cm in (16, 400):
        h = host_handle(d.num_qo_heads, d.num_kv_heads, d.head_dim, d.page_size, nwg=256, cost_mfma=cm)
        h.plan(d.qo_indptr, d.kv_indptr, d.last_page_len)
        bytes_for.append(h.plan_bytes().tobytes())
    assert bytes_for[0] == bytes_for[1]


def unit_chunks(plan, group):
    """Chunks grouped by (first token, head): list of (kv_begin, kv_end, partial)."""
    units = {}
    for it in plan["items"]:
        key = (int(it["qo_begin"]), int(it["kv_head"]), int(it["page_begin"]))
        units.setdefault(key, []).append(
            (int(it["kv_begin"]), int(it["kv_end"]), bool(it["flags"] & plan_blob.ITEM_PARTIAL))
        )
    return units


@pytest.mark.parametrize("name", ["tiny_decode_f32", "batch_decode", "skewed_long_decode", "ragged_causal_prefill"])
@pytest.mark.parametrize("nwg", [1, 64, 512])
def test_named_workload_plan_invariants(name, nwg):
    w = W.named(name, tensors=False)
    # (the plan's own assignment: every item on the workgroup it is given)
    h = host_handle(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, w.dtype, w.causal, w.cap, nwg,
                    static_queues=True)
    info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    plan = plan_blob.decode(h.plan_bytes())
    items = plan["items"]
    assert plan["header"]["pool_begin"] == len(items)
    lens = items["kv_end"] - items["kv_begin"]
    # chunks never exceed L_kv
    assert np.all(lens <= info["kv_chunk"])
    # L_kv follows the pages' formula (rounded to the 64-key granule, at least 64);
    # the planner keeps it, a refinement L_kv / k (k <= 4), or filling at L_kv
    # (pieces up to 2 L_kv), whichever predicts the smallest makespan
    g = w.group
    tile_tokens = max(1, info["q_tile"] // g)
    total = 0
    for lq, lk in zip(w.qo_lens, w.kv_lens):
        for t0 in range(0, int(lq), tile_tokens):
            nt = min(tile_tokens, int(lq) - t0)
            eff = min(int(lk), int(lk) - int(lq) + t0 + nt) if w.causal else int(lk)
            total += eff * w.num_kv_heads
    pages_lkv = max(-(-max(-(-total // nwg), 1) // 64) * 64, 64)
    candidates = {max(-(-(-(-pages_lkv // k)) // 64) * 64, 64) for k in range(1, 5)}
    filled = info["kv_chunk"] not in candidates
    if filled:
        assert pages_lkv <= info["kv_chunk"] <= 2 * pages_lkv
    # per unit: chunks tile [0, l_eff) without gaps; partial iff split
    n_split_chunks = 0
    n_split_units = 0
    for chunks in unit_chunks(plan, g).values():
        chunks.sort()
        assert chunks[0][0] == 0
        for a, b in zip(chunks, chunks[1:]):
            assert a[1] == b[0]
        split = len(chunks) > 1
        assert all(c[2] == split for c in chunks)
        n_split_chunks += len(chunks) if split else 0
        n_split_units += int(split)
    # partial-output bound of paper Appendix D.3 (2 * #workgroups chunks at the
    # pages' L_kv; at a chunk L it reads 2 * sum / L)
    if filled:
        # filling cuts about one piece per workgroup plus one tail per split unit
        assert n_split_chunks <= 2 * nwg + n_split_units
    else:
        assert n_split_chunks <= 2 * -(-total // info["kv_chunk"])
        if info["kv_chunk"] == pages_lkv:
            assert n_split_chunks <= 2 * nwg
    assert info["num_partial_items"] == n_split_chunks
    # queues are longest-first (cost = rows + keys + the fixed item cost 512);
    # with filling, the unsplit units come first, longest first; where partial
    # states are released early, a queue runs its partial items first, and each
    # part is longest-first
    for wg in range(nwg):
        q_items = items[plan["item_ptr"][wg] : plan["item_ptr"][wg + 1]]
        part = (q_items["flags"] & plan_blob.ITEM_PARTIAL) != 0
        if filled or (items["flags"] & plan_blob.ITEM_RELEASE).any():
            q_items = q_items[~part]
        cost = q_items["qo_count"] * g + (q_items["kv_end"] - q_items["kv_begin"]) + 512
        assert np.all(np.diff(cost) <= 0)
    # longest-processing-time bound on the busiest workgroup: attention items by LPT,
    # then its merge tasks, which start once their sources are ready (at the latest
    # when the attention phase ends everywhere)
    att = items["qo_count"].astype(np.int64) * g + (items["kv_end"] - items["kv_begin"]) + 512
    att_bound = att.sum() / nwg + int(att.max())
    if len(plan["merge"]):
        max_task = 512 + g * int(plan["merge"]["src_count"].max())
        tasks_per_wg = int(np.diff(plan["merge_ptr"]).max())
        assert info["max_wg_cost"] <= att_bound + tasks_per_wg * max_task
        # tasks are spread: no workgroup holds two while another holds none (when
        # every partial state is ready only at the end of its queue; states released
        # early let a workgroup that is idle by then take several)
        if len(plan["merge"]) <= nwg and not (items["flags"] & plan_blob.ITEM_RELEASE).any():
            assert tasks_per_wg == 1
    else:
        assert info["max_wg_cost"] <= att_bound
    # determinism: same lengths, same bytes; the plan never sees page ids
    first = h.plan_bytes()
    h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    assert np.array_equal(first, h.plan_bytes())
    h2 = host_handle(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, w.dtype, w.causal, w.cap, nwg,
                     static_queues=True)
    h2.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    assert np.array_equal(first, h2.plan_bytes())


def test_kernel_choice_follows_query_tile_rule():
    """Decode rows alone run on the decode body, wide rows on tiles; both together
    on the mixed grid only when the decode-sized rows stream at least a quarter of
    the KV tokens (tiles counted once per 128-row query tile), otherwise every row
    runs as a tile."""
    h = host_handle(32, 8, 128, 16, nwg=16)
    assert h.plan([0, 1, 2], [0, 1, 2], [16, 16])["kernel"] == lib.KERNEL_DECODE
    assert h.plan([0, 1, 2], [0, 1, 2], [16, 16])["q_tile"] == 4
    assert h.plan([0, 2, 3], [0, 1, 2], [16, 16])["q_tile"] == 8
    assert h.plan([0, 300], [0, 20], [16])["kernel"] == lib.KERNEL_MFMA
    # 300 tokens (10 tiles x 320 keys) and a one-token row over 16 keys: tiles only
    info = h.plan([0, 300, 301], [0, 20, 21], [16, 16])
    assert info["kernel"] == lib.KERNEL_MFMA and info["q_tile"] == 128
    # the one-token row over 1200 keys (27 % of 4400): mixed
    assert h.plan([0, 300, 301], [0, 20, 95], [16, 16])["kernel"] == lib.KERNEL_MIXED
    # over 1040 keys (24.5 %): tiles
    assert h.plan([0, 300, 301], [0, 20, 85], [16, 16])["kernel"] == lib.KERNEL_MFMA


@pytest.mark.parametrize(
    "qo, kv, last, causal, code",
    [
        ([0, 1, 0], [0, 1, 2], [3, 3], False, lib.BSR_ERR_INVALID_ARG),    # qo_indptr decreasing
        ([0, 1, 2], [0, 2, 1], [3, 3], False, lib.BSR_ERR_INVALID_ARG),    # kv_indptr decreasing
        ([0, 1, 2], [0, 1, 2], [0, 3], False, lib.BSR_ERR_INVALID_ARG),    # last_page_len < 1
        ([0, 1, 2], [0, 1, 2], [3, 17], False, lib.BSR_ERR_INVALID_ARG),   # last_page_len > P
        ([0, 5, 6], [0, 1, 2], [3, 3], True, lib.BSR_ERR_INVALID_ARG),     # causal l_qo > l_kv
        ([1, 2, 3], [0, 1, 2], [3, 3], False, lib.BSR_ERR_INVALID_ARG),    # qo_indptr[0] != 0
    ],
)
def test_plan_rejects_malformed(qo, kv, last, causal, code):
    h = host_handle(8, 2, 64, 16, causal=causal)
    with pytest.raises(lib.BsrError) as e:
        h.plan(qo, kv, last)
    assert e.value.code == code


def test_plan_capacity_errors():
    h = host_handle(8, 2, 64, 16, max_batch=2, max_total_qo=4, max_total_kv=100)
    with pytest.raises(lib.BsrError) as e:
        h.plan([0, 1, 2, 3], [0, 1, 2, 3], [1, 1, 1])
    assert e.value.code == lib.BSR_ERR_CAPACITY
    with pytest.raises(lib.BsrError) as e:
        h.plan([0, 5], [0, 1], [1])
    assert e.value.code == lib.BSR_ERR_CAPACITY
    with pytest.raises(lib.BsrError) as e:
        h.plan([0, 1], [0, 7], [16])
    assert e.value.code == lib.BSR_ERR_CAPACITY


def test_empty_batch_plans():
    h = host_handle(8, 2, 64, 16)
    info = h.plan([0], [0], [])
    assert info["num_items"] == 0 and info["num_merge_tasks"] == 0


WINDOW_CASES = [
    # name, qo_lens, kv_lens, h_qo, h_kv, d, P, dtype, causal, nwg, window
    ("decode_window_split", [1, 1, 1, 1], [17, 640, 1000, 2550], 8, 2, 64, 16, "f32", False, 16, 300),
    ("prefill_causal_window", [40, 7, 300], [100, 7, 900], 8, 2, 64, 1, "bf16", True, 8, 129),
    ("noncausal_window", [33, 1], [90, 450], 4, 1, 64, 2, "bf16", False, 5, 64),
    ("window_one", [5, 1, 2], [5, 70, 200], 4, 2, 64, 3, "bf16", True, 4, 1),
    ("window_covers_all", [3, 1], [50, 90], 4, 2, 64, 16, "bf16", True, 4, 1000),
    ("window_empty_rows", [1, 0, 1, 2], [0, 5, 70, 0], 4, 2, 64, 4, "bf16", False, 4, 10),
    # more queries than keys (non-causal) and the largest window: no int32 overflow
    ("window_huge_noncausal", [9, 1], [4, 70], 4, 2, 64, 3, "bf16", False, 4, 2**31 - 1),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=[c[0] for c in WINDOW_CASES])
def test_window_plan_executes_to_oracle(case):
    """A sliding-window plan reproduces the oracle's windowed attention, and its
    items read no key below the first token's window (rounded down to the 64-key
    chunk granule)."""
    name, qo, kv, h_qo, h_kv, d, P, dtype, causal, nwg, window = case
    w = W.build(name, 8, qo, kv, P, h_qo, h_kv, d, dtype=dtype, causal=causal, window=window)
    h = host_handle(h_qo, h_kv, d, P, dtype, causal, 0.0, nwg, sliding_window=window)
    h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    plan = plan_blob.decode(h.plan_bytes())
    q, k, v = f64(w.q), f64(w.k_pool), f64(w.v_pool)
    o, lse, written = plan_blob.execute(plan, q, k, v, w.kv_indices, w.group, P, w.scale, 0.0)
    ro, rl = oracle.bsr_attention(q, k, v, w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, P, h_qo, h_kv,
                                  w.scale, causal, 0.0, window)
    assert np.all(written == 1)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], rl[fin], rtol=1e-12, atol=1e-12)
    qo_ptr = np.asarray(w.qo_indptr)
    for it in plan["items"]:
        r = int(np.searchsorted(qo_ptr, int(it["qo_begin"]), side="right")) - 1
        t0 = int(it["qo_begin"]) - int(qo_ptr[r])
        first = kv[r] - qo[r] + t0 - window + 1
        assert int(it["window_lo"]) == max(first, -0x3FFFFFFF)
        assert int(it["kv_begin"]) >= max(first, 0) // 64 * 64, name


def test_window_shortens_long_decode_plans():
    """Decode over 4096 keys with a 256-key window plans about 256 keys per request."""
    qo, kv = [1] * 4, [4096] * 4
    w = W.build("window_decode", 9, qo, kv, 16, 8, 2, 64, tensors=False)
    h = host_handle(8, 2, 64, 16, "bf16", True, 0.0, 8, sliding_window=256)
    h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    plan = plan_blob.decode(h.plan_bytes())
    keys = sum(int(it["kv_end"]) - int(it["kv_begin"]) for it in plan["items"])
    assert keys <= 4 * 2 * (256 + 64), keys


def test_composable_plan_rejects_window():
    h = host_handle(8, 2, 64, 16, sliding_window=16)
    fmt = dict(qo_indptr=np.array([0, 1], dtype=np.int32), kv_indptr=np.array([0, 1], dtype=np.int32),
               last_page_len=np.array([4], dtype=np.int32), kv_indices_offset=0)
    with pytest.raises(lib.BsrError) as e:
        h.plan_composable([fmt], 1)
    assert e.value.code == lib.BSR_ERR_UNSUPPORTED


def test_create_rejects_negative_window():
    with pytest.raises(lib.BsrError) as e:
        host_handle(8, 2, 64, 16, sliding_window=-1)
    assert e.value.code == lib.BSR_ERR_INVALID_ARG


def test_window_batch_is_balanced_by_the_half_chunk_fill():
    """Under a 4096-key window most decode units are a little over L_kv / 2 long;
    whole units would leave workgroups with two of them (max/mean 1.17).  The plan
    cuts some of them and stays within 10 % of the mean."""
    w = W.named("batch_decode_window", tensors=False)
    h = host_handle(32, 8, 128, 16, "bf16", False, 0.0, 256, max_batch=64, sliding_window=w.window)
    info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    assert info["num_partial_items"] > 0
    assert info["max_wg_cost"] <= 1.10 * info["total_cost"] / 256
