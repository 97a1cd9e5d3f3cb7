"""Claimed work items (the default layout of MFMA tile plans): the tail of each
workgroup's queue (items starting after 7/8 of its planned load, never its first
item) goes to a pool that free workgroups claim at run time, longest first.  The items themselves, the partial
states and the merge map are those of the static plan, so both layouts compute
the same thing; the executor runs every item once either way."""

import numpy as np
import pytest

from serving_attention_bsr_amd import lib
from serving_attention_bsr_amd import workloads as W
from tests import plan_blob


def plan_of(w, nwg, static_queues, composable=False):
    mb = w.batch + (sum(len(f.qo_indptr) - 1 for f in w.formats) if composable else 0)
    h = lib.BsrAttention(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, dtype=w.dtype, causal=w.causal,
                         logits_soft_cap=w.cap, num_workgroups=nwg, device=-1, max_batch=mb,
                         max_total_qo=int(w.qo_indptr[-1]), max_total_kv=int(w.kv_lens.sum()) + 64,
                         static_queues=static_queues)
    if composable:
        info = h.plan_composable([f.as_dict() for f in w.formats], w.batch)
    else:
        info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    return info, plan_blob.decode(h.plan_bytes())


def item_set(items):
    fields = [f for f in items.dtype.names if not f.startswith("pad")]
    return sorted(tuple(int(it[f]) for f in fields) for it in items)


@pytest.mark.parametrize("name, nwg", [("batch_decode", 256), ("skewed_long_decode", 256),
                                       ("ragged_causal_prefill", 512), ("batch_decode", 7)])
def test_pool_holds_the_queue_tails_longest_first(name, nwg):
    w = W.named(name, tensors=False)
    info_s, st = plan_of(w, nwg, True)
    info_d, dy = plan_of(w, nwg, False)
    # same items, partial states and merges; only their placement differs
    assert item_set(st["items"]) == item_set(dy["items"])
    assert info_s["num_partial_items"] == info_d["num_partial_items"]
    assert np.array_equal(st["srcs"], dy["srcs"]) and len(st["merge"]) == len(dy["merge"])
    # static: no pool; claimed: each queue is a prefix of the static queue, and the
    # pool holds the rest, longest first
    assert st["header"]["pool_begin"] == len(st["items"])
    pool_begin = dy["header"]["pool_begin"]
    ptr_s, ptr_d = st["item_ptr"], dy["item_ptr"]
    assert ptr_d[-1] == pool_begin
    g = w.group
    cost = lambda it: it["qo_count"].astype(np.int64) * g + (it["kv_end"] - it["kv_begin"])
    for wg in range(nwg):
        qs = st["items"][ptr_s[wg]:ptr_s[wg + 1]]
        qd = dy["items"][ptr_d[wg]:ptr_d[wg + 1]]
        assert len(qd) >= min(len(qs), 1)
        assert qd.tobytes() == qs[:len(qd)].tobytes()
        # what left the queue is its tail: it starts after 7/8 of the queue's cost
        # (the planner's cost adds a fixed cost per item)
        if len(qd) < len(qs):
            c = cost(qs) + 512
            assert c[:len(qd)].sum() * 16 >= c.sum() * 14
    pool = dy["items"][pool_begin:]
    assert np.all(np.diff(cost(pool)) <= 0)
    assert np.all(dy["claims"] == 0)


def test_composable_pool_keeps_the_merge_map():
    w = W.shared_prefix_composable(tensors=False)
    info_s, st = plan_of(w, 256, True, composable=True)
    info_d, dy = plan_of(w, 256, False, composable=True)
    assert item_set(st["items"]) == item_set(dy["items"])
    assert np.array_equal(st["srcs"], dy["srcs"])
    # a mixed grid keeps its queues
    assert dy["header"]["pool_begin"] == len(dy["items"])


def test_pool_only_for_tile_grids():
    """Decode grids keep their queues (no pool); the ragged prefill on the MFMA
    tile grid, about a dozen items per workgroup, pools its queue tails."""
    for name, nwg, pooled in (("batch_decode", 256, False), ("skewed_long_decode", 256, False),
                              ("ragged_causal_prefill", 512, True)):
        w = W.named(name, tensors=False)
        info, p = plan_of(w, nwg, False)
        n_pool = info["num_items"] - p["header"]["pool_begin"]
        assert (n_pool > 0) == pooled, (name, n_pool)


def test_create_rejects_bad_static_queues():
    with pytest.raises(lib.BsrError) as e:
        lib.BsrAttention(8, 2, 64, 16, num_workgroups=4, device=-1, max_batch=4, max_total_qo=4, max_total_kv=64,
                         static_queues=2)
    assert e.value.code == lib.BSR_ERR_INVALID_ARG
