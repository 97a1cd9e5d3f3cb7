"""Determinism, graph capture and the error paths of run() on the MFMA and mixed
kernels (needs an MI355X).

* The same plan gives the same bits on every run (the contraction of partial
  states follows the plan's fixed order, no atomics: Core mechanism 6 of the
  FlashInfer explainer page, paper Algorithm 1), at full size, for the MFMA tile
  kernel (ragged causal prefill) and the mixed kernel (shared-prefix composed
  formats).
* A run captured in a HIP graph replays later plans made for the same kernel
  instance (Core mechanism 7, paper Appendix D): capture, re-plan new lengths,
  replay, compare with the oracle, for the MFMA and mixed kinds.
* A replay that meets a plan made for another instance computes nothing and
  check() reports it; a merge whose wait for a ready stamp expires (forced from
  the host: a stamp no item writes and a small wait bound in the uploaded plan)
  ends normally and check() reports it.
* A plan made without a workspace leaves the uploaded plan in force.
* Items claimed at run time and items on their planned workgroups give the same
  bits (the named parity tests check the claimed layout, the default, against
  the oracle).
"""

import numpy as np
import pytest
import torch

from serving_attention_bsr_amd import lib
from serving_attention_bsr_amd import workloads as W
from tests import plan_blob
from tests.gpu_common import compare, handle_for, oracle_of, run_gpu, say, to_gpu

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).clone()


def _repeat_bitwise(w, composable, runs=10, merge=True, **kw):
    h = handle_for(w, **kw)
    q, k, v, idx = to_gpu(w)
    if composable:
        info = h.plan_composable([f.as_dict() for f in w.formats], w.batch)
        idx = torch.from_numpy(np.ascontiguousarray(w.kv_indices_formats)).to(q.device)
    else:
        info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    say("plan", info)
    if merge:
        assert info["num_partial_items"] > 0, "the case must exercise the merge"
    o, lse = h.run(q, k, v, idx)
    o0, l0 = _bits(o), _bits(lse)
    for rep in range(runs):
        o.fill_(0)
        lse.fill_(0)
        h.run(q, k, v, idx, o, lse)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o), o0), f"O differs on run {rep}"
        assert torch.equal(_bits(lse), l0), f"LSE differs on run {rep}"
    h.check()
    return info


def test_prefill_full_size_repeats_bitwise():
    """The full-size plan (6272 tiles on two workgroups per CU) needs no split."""
    say("workload ragged_causal_prefill x10")
    w = W.named("ragged_causal_prefill")
    info = _repeat_bitwise(w, False, merge=False)
    assert info["kernel"] == lib.KERNEL_MFMA


def test_split_prefill_repeats_bitwise():
    """A prefill with a long cached prefix on the default grid: long tiles are split
    and merged."""
    say("split prefill x10")
    w = W.build("split_prefill", 48, [300, 64, 1000], [700, 9000, 1500], 1, 32, 8, 128, dtype="bf16", causal=True)
    info = _repeat_bitwise(w, False)
    assert info["kernel"] == lib.KERNEL_MFMA and info["num_merge_tasks"] > 0


def test_composable_full_size_repeats_bitwise():
    say("workload shared_prefix_composable x10")
    w = W.named("shared_prefix_composable")
    info = _repeat_bitwise(w, True)
    assert info["kernel"] == lib.KERNEL_MIXED and info["num_merge_tasks"] > 0


def _graph_replan(w1, w2, composable, **kw):
    """Capture run() on w1's plan, re-plan w2 into the same workspace, replay; both
    replays must match the oracle, and w1's replays the eager run bit for bit."""
    dev = torch.device("cuda:0")
    n_pages = max(w1.k_pool.shape[0], w2.k_pool.shape[0])
    idx_of = lambda w: w.kv_indices_formats if composable else w.kv_indices
    n_idx = max(len(idx_of(w1)), len(idx_of(w2)))
    n_q = max(w1.q.shape[0], w2.q.shape[0])
    q = torch.zeros((n_q,) + tuple(w1.q.shape[1:]), dtype=w1.q.dtype, device=dev)
    k = torch.empty((n_pages,) + tuple(w1.k_pool.shape[1:]), dtype=w1.k_pool.dtype, device=dev)
    v = torch.empty_like(k)
    idx = torch.zeros(n_idx, dtype=torch.int32, device=dev)
    o = torch.zeros_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=dev)
    mb = max(w.batch + (sum(len(f.qo_indptr) - 1 for f in w.formats) if composable else 0) for w in (w1, w2))
    h = handle_for(w1, max_batch=mb, max_total_qo=n_q, max_total_kv=int(max(w1.kv_lens.sum(), w2.kv_lens.sum())),
                   **kw)

    def load(w):
        q[: w.q.shape[0]].copy_(w.q)
        k[: w.k_pool.shape[0]].copy_(w.k_pool)
        v[: w.v_pool.shape[0]].copy_(w.v_pool)
        idx[: len(idx_of(w))].copy_(torch.from_numpy(np.ascontiguousarray(idx_of(w))))
        if composable:
            info = h.plan_composable([f.as_dict() for f in w.formats], w.batch)
        else:
            info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
        torch.cuda.synchronize()
        say("plan", info)
        return info

    i1 = load(w1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        h.run(q, k, v, idx, o, lse)  # warm the launch path outside capture
    torch.cuda.synchronize()
    eager_o, eager_l = _bits(o), _bits(lse)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        h.run(q, k, v, idx, o, lse)
    n1 = w1.q.shape[0]
    ro, rl = oracle_of(w1, composable)
    for rep in range(3):
        o.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(o), eager_o) and torch.equal(_bits(lse), eager_l), f"replay {rep} differs from eager"
        compare(w1, o[:n1].double().cpu().numpy(), lse[:n1].double().cpu().numpy(), ro, rl, f"graph replay {rep}")
    i2 = load(w2)
    assert (i2["kernel"], i2["instance"], i2["num_workgroups"]) == (i1["kernel"], i1["instance"], i1["num_workgroups"])
    n2 = w2.q.shape[0]
    ro2, rl2 = oracle_of(w2, composable)
    for rep in range(2):
        o.zero_()
        g.replay()
        torch.cuda.synchronize()
        compare(w2, o[:n2].double().cpu().numpy(), lse[:n2].double().cpu().numpy(), ro2, rl2, f"replan replay {rep}")
    h.check()
    return i1, i2


def test_graph_replays_mfma_plans_across_a_replan():
    mk = lambda seed, qo, kv: W.build(f"prefill_{seed}", seed, qo, kv, 1, 32, 8, 128, dtype="bf16", causal=True)
    w1 = mk(41, [64, 100], [6000, 3000])
    w2 = mk(42, [40, 130], [8000, 2000])
    i1, i2 = _graph_replan(w1, w2, False, num_workgroups=64)
    assert i1["kernel"] == lib.KERNEL_MFMA and i1["num_partial_items"] > 0 and i2["num_partial_items"] > 0


def test_graph_replays_mixed_plans_across_a_replan():
    mk = lambda seed, branches, prefix: W.shared_prefix_composable(seed=seed, branches=branches, prefix_len=prefix,
                                                                   suf_lo=20, suf_hi=300)
    w1 = mk(43, 16, 2048)
    w2 = mk(44, 24, 1024)
    i1, i2 = _graph_replan(w1, w2, True)
    assert i1["kernel"] == lib.KERNEL_MIXED and i1["num_merge_tasks"] > 0 and i2["num_merge_tasks"] > 0


def test_prefill_page_permutation_keeps_bits():
    """One-key pages: a physical permutation of the pool's slots (page ids remapped
    accordingly) gives the same bits, on the split MFMA plan."""
    w = W.build("perm_p1", 45, [64, 33], [5000, 2000], 1, 32, 8, 128, dtype="bf16", causal=True)
    o, lse, info = run_gpu(w, num_workgroups=64)
    assert info["kernel"] == lib.KERNEL_MFMA and info["num_partial_items"] > 0
    perm = np.random.default_rng(6).permutation(w.k_pool.shape[0])
    inv = np.argsort(perm)
    w2 = W.build("perm_p1", 45, [64, 33], [5000, 2000], 1, 32, 8, 128, dtype="bf16", causal=True)
    w2.k_pool = w.k_pool[torch.from_numpy(inv)]
    w2.v_pool = w.v_pool[torch.from_numpy(inv)]
    w2.kv_indices = perm[w.kv_indices].astype(np.int32)
    o2, lse2, _ = run_gpu(w2, num_workgroups=64)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_replay_of_another_instance_is_reported():
    """Capture a one-token decode (4 folded rows), re-plan with a two-token request
    (8 rows, another instance): the replay computes nothing and check() reports
    it; the re-uploaded plan then runs eagerly and matches the oracle."""
    w1 = W.build("spec1", 46, [1] * 8, [100, 2000, 37, 900, 512, 4000, 1, 64], 16, 32, 8, 128, dtype="bf16")
    w2 = W.build("spec2", 46, [2] + [1] * 7, [100, 2000, 37, 900, 512, 4000, 1, 64], 16, 32, 8, 128, dtype="bf16")
    dev = torch.device("cuda:0")
    q = torch.zeros((w2.q.shape[0],) + tuple(w2.q.shape[1:]), dtype=w2.q.dtype, device=dev)
    k, v = w2.k_pool.to(dev), w2.v_pool.to(dev)
    idx = torch.from_numpy(np.ascontiguousarray(w2.kv_indices)).to(dev)
    o = torch.zeros_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=dev)
    h = handle_for(w2)
    q[: w1.q.shape[0]].copy_(w1.q)
    i1 = h.plan(w1.qo_indptr, w1.kv_indptr, w1.last_page_len)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        h.run(q, k, v, idx, o, lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        h.run(q, k, v, idx, o, lse)
    q.copy_(w2.q)
    i2 = h.plan(w2.qo_indptr, w2.kv_indptr, w2.last_page_len)
    torch.cuda.synchronize()
    say("instances", i1["instance"], i2["instance"])
    assert i1["instance"] != i2["instance"]
    o.fill_(7.0)
    g.replay()
    torch.cuda.synchronize()
    with pytest.raises(lib.BsrError) as e:
        h.check()
    assert e.value.code == lib.BSR_ERR_DEVICE and "instance" in str(e.value)
    assert bool(torch.all(o == 7.0)), "a refused plan writes no output"
    h.plan(w2.qo_indptr, w2.kv_indptr, w2.last_page_len)  # fresh upload: status words cleared
    h.run(q, k, v, idx, o, lse)
    torch.cuda.synchronize()
    h.check()
    ro, rl = oracle_of(w2)
    compare(w2, o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, "8-row plan, eager")


def test_expired_merge_wait_is_reported():
    """A merge source whose ready stamp no item writes: the merge's bounded wait
    (shortened in the uploaded plan) expires, every workgroup ends, check()
    returns BSR_ERR_DEVICE; a fresh upload then runs clean."""
    w = W.named("skewed_long_decode", long_len=16384, n_short=7)
    h = handle_for(w, num_workgroups=64)
    q, k, v, idx = to_gpu(w)
    info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    assert info["num_partial_items"] >= 2
    torch.cuda.synchronize()
    blob = h.plan_bytes().copy()
    plan = plan_blob.decode(blob)
    hdr = plan["header"]
    items = plan["items"]
    part = np.nonzero(items["flags"] & plan_blob.ITEM_PARTIAL)[0]
    a, b = int(part[0]), int(part[1])
    assert items["flag_id"][a] != items["flag_id"][b]
    # item a stamps item b's flag instead of its own: a's flag is never written
    item_off = hdr["off_items"] + a * plan_blob.ITEM.itemsize + plan_blob.ITEM.fields["flag_id"][1]
    blob[item_off:item_off + 4] = np.frombuffer(np.int32(items["flag_id"][b]).tobytes(), dtype=np.uint8)
    spin_off = 4 * plan_blob.HEADER_FIELDS.index("spin_limit")
    blob[spin_off:spin_off + 4] = np.frombuffer(np.int32(2000).tobytes(), dtype=np.uint8)
    h.workspace[: len(blob)].copy_(torch.from_numpy(blob))
    torch.cuda.synchronize()
    h.run(q, k, v, idx)
    torch.cuda.synchronize()
    with pytest.raises(lib.BsrError) as e:
        h.check()
    assert e.value.code == lib.BSR_ERR_DEVICE and "waiting" in str(e.value)
    o, lse, _ = run_gpu(w, h=h)
    ro, rl = oracle_of(w)
    compare(w, o, lse, ro, rl, "after a fresh upload")


def test_plan_without_workspace_keeps_the_uploaded_plan():
    """bsr_attn_plan with a null workspace stages a plan without uploading it: run()
    keeps launching the uploaded one (and its kernel instance)."""
    w1 = W.build("up1", 47, [1] * 4, [300, 20, 1000, 77], 16, 32, 8, 128, dtype="bf16")
    w2 = W.build("up2", 47, [2, 1, 1, 1], [300, 20, 1000, 77], 16, 32, 8, 128, dtype="bf16")
    h = handle_for(w2)
    q, k, v, idx = to_gpu(w1)
    h.plan(w1.qo_indptr, w1.kv_indptr, w1.last_page_len)
    o1, l1 = h.run(q, k, v, idx)
    torch.cuda.synchronize()
    o1, l1 = _bits(o1), _bits(l1)
    lib.bsr_attn_plan(h.handle, w2.qo_indptr, w2.kv_indptr, w2.last_page_len, None, h._staging_ptr, h._stream())
    assert h.info()["q_tile"] == 8  # the staged plan is w2's
    o, l = h.run(q, k, v, idx)
    torch.cuda.synchronize()
    h.check()
    assert torch.equal(_bits(o), o1) and torch.equal(_bits(l), l1)


def _outputs(w, composable, **kw):
    h = handle_for(w, **kw)
    q, k, v, idx = to_gpu(w)
    if composable:
        info = h.plan_composable([f.as_dict() for f in w.formats], w.batch)
        idx = torch.from_numpy(np.ascontiguousarray(w.kv_indices_formats)).to(q.device)
    else:
        info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    o, lse = h.run(q, k, v, idx)
    torch.cuda.synchronize()
    h.check()
    return info, _bits(o), _bits(lse)


@pytest.mark.parametrize("name, nwg", [("split_prefill", 64), ("ragged_causal_prefill", 0)])
def test_claimed_items_match_the_static_queues_bitwise(name, nwg):
    """Work items claimed at run time (the default on the MFMA tile grid) and every
    item on the workgroup the plan names give the same bits: the items, partial
    states and merge order are the same; only which workgroup runs an item
    differs.  (The split prefill on 64 workgroups has long queues and merges.)"""
    say("claimed vs static queues", name, nwg)
    if name == "split_prefill":
        w = W.build("split_prefill", 48, [300, 64, 1000], [700, 9000, 1500], 1, 32, 8, 128, dtype="bf16",
                    causal=True)
    else:
        w = W.named(name)
    info_d, o_d, l_d = _outputs(w, False, num_workgroups=nwg)
    info_s, o_s, l_s = _outputs(w, False, num_workgroups=nwg, static_queues=True)
    say("plans", info_d["num_items"], info_d["num_partial_items"], info_s["num_items"])
    assert info_d["kernel"] == lib.KERNEL_MFMA and info_d["num_items"] == info_s["num_items"]
    if name == "split_prefill":
        assert info_d["num_partial_items"] > 0
    assert torch.equal(o_d, o_s) and torch.equal(l_d, l_s)
