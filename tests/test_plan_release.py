"""Early release of partial states (Core mechanism 6 of the FlashInfer explainer
page, paper Algorithm 1: merges wait on ready stamps).  In decode and mixed grids
each workgroup runs its items that write partial states first, and every such item
that is not the last of its queue is stamped right after it, so that a merge can
run while the queue's direct items go on.  Tile grids (claimed queue tails) and
composed formats keep one stamp pass per queue."""

import numpy as np

from serving_attention_bsr_amd import lib
from serving_attention_bsr_amd import workloads as W
from tests import plan_blob


def plan_of(w, nwg, composable=False):
    mb = w.batch + (sum(len(f.qo_indptr) - 1 for f in w.formats) if composable else 0)
    h = lib.BsrAttention(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, dtype=w.dtype, causal=w.causal,
                         logits_soft_cap=w.cap, num_workgroups=nwg, device=-1, max_batch=mb,
                         max_total_qo=int(w.qo_indptr[-1]), max_total_kv=int(w.kv_lens.sum()) + 64)
    if composable:
        info = h.plan_composable([f.as_dict() for f in w.formats], w.batch)
    else:
        info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    return info, plan_blob.decode(h.plan_bytes())


def test_skewed_batch_releases_the_long_chunks_early():
    w = W.named("skewed_long_decode", tensors=False)
    info, p = plan_of(w, 256)
    assert info["kernel"] == 1
    its, ptr = p["items"], p["item_ptr"]
    part = (its["flags"] & plan_blob.ITEM_PARTIAL) != 0
    rel = (its["flags"] & plan_blob.ITEM_RELEASE) != 0
    assert rel.any()
    assert not (rel & ~part).any()  # only partial states are released
    for wg in range(256):
        q = slice(ptr[wg], ptr[wg + 1])
        qp, qr = part[q], rel[q]
        if len(qp) == 0:
            continue
        # partial items first, then direct ones
        assert not np.any(np.diff(qp.astype(int)) > 0)
        # every partial item but the queue's last is released early
        expect = qp.copy()
        expect[-1] = False
        assert np.array_equal(qr, expect)
    # the flags of the released states are still those the merges wait on
    srcs = {int(s["flag_id"]) for s in p["srcs"]}
    assert {int(f) for f in its["flag_id"][rel]} <= srcs


def test_tile_grids_and_composed_formats_keep_one_stamp_pass():
    for name, comp in (("ragged_causal_prefill", False), ("shared_prefix_composable", True)):
        w = W.named(name, tensors=False)
        _, p = plan_of(w, 64, composable=comp)
        assert not (p["items"]["flags"] & plan_blob.ITEM_RELEASE).any()
