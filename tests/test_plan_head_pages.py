"""Plans over one page list per request and KV head (the output of the Quest
page choice), through a host-only handle: the CPU float64 executor must
reproduce attention over each head's own keys, computed with the oracle's plain
attention over explicitly gathered keys."""

import numpy as np
import pytest

import oracle
from serving_attention_bsr_amd import lib
from serving_attention_bsr_amd import workloads as W
from tests import plan_blob


def per_head_lists(w, keep, seed):
    """For each (request, KV head) a subset of the request's pages, in logical order,
    always ending with its last page; returns kv_indptr [B H_kv + 1], kv_indices,
    and the logical positions kept."""
    rng = np.random.default_rng(seed)
    ptr, ids, kept = [0], [], []
    for r in range(w.batch):
        b, e = int(w.kv_indptr[r]), int(w.kv_indptr[r + 1])
        n = e - b
        row = []
        for h in range(w.num_kv_heads):
            if n <= keep:
                pos = np.arange(n)
            else:
                pos = np.sort(np.concatenate([rng.choice(n - 1, keep - 1, replace=False), [n - 1]]))
            ids += list(w.kv_indices[b + pos])
            ptr.append(ptr[-1] + len(pos))
            row.append(pos)
        kept.append(row)
    return np.array(ptr, dtype=np.int32), np.array(ids, dtype=np.int32), kept


def reference(w, kept):
    q, k, v = w.q.double().numpy(), w.k_pool.double().numpy(), w.v_pool.double().numpy()
    g = w.group
    out = np.zeros(q.shape)
    lse = np.full(q.shape[:2], -np.inf)
    for r in range(w.batch):
        b, e = int(w.kv_indptr[r]), int(w.kv_indptr[r + 1])
        t0, t1 = int(w.qo_indptr[r]), int(w.qo_indptr[r + 1])
        for hk in range(w.num_kv_heads):
            kk, vv = [], []
            for p in kept[r][hk]:
                valid = w.page_size if b + p < e - 1 else int(w.last_page_len[r])
                page = int(w.kv_indices[b + p])
                kk.append(k[page, hk, :valid])
                vv.append(v[page, hk, :valid])
            kk = np.concatenate(kk) if kk else np.zeros((0, w.head_dim))
            vv = np.concatenate(vv) if vv else np.zeros((0, w.head_dim))
            for j in range(g):
                h = hk * g + j
                o1, l1 = oracle.attention_dense(q[t0:t1, h], kk, vv, w.scale, w.cap)
                out[t0:t1, h] = o1
                lse[t0:t1, h] = l1
    return out, lse


@pytest.mark.parametrize("nwg, keep, P, h_qo, h_kv", [(8, 3, 16, 8, 2), (16, 5, 4, 4, 4), (4, 100, 3, 8, 4)])
def test_head_page_plan_executes_to_reference(nwg, keep, P, h_qo, h_kv):
    w = W.build("heads", 23, [1, 1, 1, 1], [170, 16, 1, 900], P, h_qo, h_kv, 64, cap=4.0)
    ptr, ids, kept = per_head_lists(w, keep, 24)
    h = lib.BsrAttention(h_qo, h_kv, 64, P, num_workgroups=nwg, device=-1, max_batch=8, max_total_qo=8,
                         max_total_kv=1 << 12, logits_soft_cap=4.0)
    h.plan_head_pages(w.qo_indptr, ptr, w.last_page_len)
    plan = plan_blob.decode(h.plan_bytes())
    o, lse, written = plan_blob.execute(plan, w.q.double().numpy(), w.k_pool.double().numpy(),
                                        w.v_pool.double().numpy(), ids, w.group, P, w.scale, 4.0)
    ro, rl = reference(w, kept)
    assert np.all(written == 1)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


def test_head_page_plan_rejects_bad_tables():
    h = lib.BsrAttention(4, 2, 64, 16, num_workgroups=4, device=-1, max_batch=4, max_total_qo=4, max_total_kv=1024)
    with pytest.raises(lib.BsrError) as e:
        h.plan_head_pages([0, 1], [0, 2, 1], [5])  # decreasing per-head indptr
    assert e.value.code == lib.BSR_ERR_INVALID_ARG
    with pytest.raises(lib.BsrError) as e:
        h.plan_head_pages([0, 1], [0, 1, 2], [17])  # last_page_len > P
    assert e.value.code == lib.BSR_ERR_INVALID_ARG
