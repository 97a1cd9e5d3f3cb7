"""Pins of the Quest-style page-budget oracle (oracle/quest.py).

Each pin takes the quest module and raises on a mismatch.  The anchors are
mathematical: the summaries bound every key of their page and are attained; a
page's score bounds q.k over its keys from above and is exact for a one-key page;
the kept pages of each request and KV head are a valid top set (no dropped page
outscores a kept one, the last page is kept, ties go to the earlier page); a
crafted cache whose best pages are known by construction; a budget that keeps
every page reproduces plain attention; and the attention over the kept keys
equals a term-by-term softmax with math.exp over an explicit key list.
"""

from __future__ import annotations

import math

import numpy as np


def _case(seed, kv_lens, page_size, h_qo, h_kv, d):
    rng = np.random.default_rng(seed)
    n_pages = [(l + page_size - 1) // page_size for l in kv_lens]
    num_pages = sum(n_pages) + 3
    kv_indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int64)
    kv_indices = rng.permutation(num_pages)[: sum(n_pages)]
    last = np.array([l - (n - 1) * page_size if n else page_size for l, n in zip(kv_lens, n_pages)])
    b = len(kv_lens)
    qo_indptr = np.arange(b + 1)
    q = rng.standard_normal((b, h_qo, d))
    k = rng.standard_normal((num_pages, h_kv, page_size, d))
    v = rng.standard_normal((num_pages, h_kv, page_size, d))
    return q, k, v, qo_indptr, kv_indptr, kv_indices, last


def _page_keys(k, kv_indptr, kv_indices, last, P, r, i):
    """The valid keys of the i-th page of request r: [H_kv, valid, D]."""
    b, e = int(kv_indptr[r]), int(kv_indptr[r + 1])
    valid = P if b + i < e - 1 else int(last[r])
    return k[int(kv_indices[b + i]), :, :valid, :]


def pin_summaries_bound_their_keys(qm):
    kv, P, h_kv, d = [37, 16, 5], 8, 2, 6
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(31, kv, P, 2, h_kv, d)
    k[:, :, -1, :] = 1e9  # slots past a last page's length must not count
    kmin, kmax = qm.page_summaries(k, kv_indptr, kv_indices, last, P)
    for r in range(len(kv)):
        for i in range(int(kv_indptr[r + 1] - kv_indptr[r])):
            keys = _page_keys(k, kv_indptr, kv_indices, last, P, r, i)
            page = int(kv_indices[kv_indptr[r] + i])
            for h in range(h_kv):
                for c in range(d):
                    col = [float(x) for x in keys[h, :, c]]
                    assert kmin[page, h, c] == min(col) and kmax[page, h, c] == max(col), (r, i, h, c)


def pin_score_bounds_every_key_and_is_exact_for_one_key(qm):
    kv, P, h_qo, h_kv, d = [50, 33, 1], 8, 4, 2, 5
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(32, kv, P, h_qo, h_kv, d)
    kmin, kmax = qm.page_summaries(k, kv_indptr, kv_indices, last, P)
    g = h_qo // h_kv
    for r in range(len(kv)):
        b, e = int(kv_indptr[r]), int(kv_indptr[r + 1])
        ids = np.asarray(kv_indices[b:e])
        sc = qm.page_scores(q[r], kmin[ids], kmax[ids], g)
        for i in range(e - b):
            keys = _page_keys(k, kv_indptr, kv_indices, last, P, r, i)
            for hk in range(h_kv):
                best = max(sum(float(a) * float(x) for a, x in zip(q[r, h], key))
                           for h in range(hk * g, hk * g + g) for key in keys[hk])
                assert sc[hk, i] >= best - 1e-12, (r, i, hk)
                if keys.shape[1] == 1:
                    assert abs(sc[hk, i] - best) < 1e-12, (r, i, hk)


def pin_kept_pages_are_a_valid_top_set(qm):
    kv, P, h_qo, h_kv, d, budget = [300, 90, 40, 17], 4, 4, 2, 8, 6
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(33, kv, P, h_qo, h_kv, d)
    kmin, kmax = qm.page_summaries(k, kv_indptr, kv_indices, last, P)
    sel = qm.quest_selection(q, kmin, kmax, qo_indptr, kv_indptr, kv_indices, h_qo, h_kv, budget)
    for r in range(len(kv)):
        b, e = int(kv_indptr[r]), int(kv_indptr[r + 1])
        n = e - b
        ids = np.asarray(kv_indices[b:e])
        sc = qm.page_scores(q[r], kmin[ids], kmax[ids], h_qo // h_kv)
        for hk in range(h_kv):
            s = list(sel[r][hk])
            assert s == sorted(s) and len(set(s)) == len(s)
            assert len(s) == min(n, budget)
            assert s[-1] == n - 1, "the last page is kept, last"
            kept = set(s[:-1]) if n > budget else set()
            for i in range(n - 1):
                if n > budget and i not in kept:
                    for j in kept:
                        assert sc[hk, j] > sc[hk, i] or (sc[hk, j] == sc[hk, i] and j < i), (r, hk, i, j)


def pin_crafted_best_pages(qm):
    """Ten pages of four keys: pages 2 and 6 hold keys along q, the rest against it;
    a budget of 3 keeps pages 2, 6 and the last page (9)."""
    P, d = 4, 4
    q = np.array([[[1.0, 0.5, -0.25, 2.0]]])
    k = np.zeros((12, 1, P, d))
    for p in range(12):
        k[p, 0] = -np.abs(q[0, 0])[None, :] * np.sign(q[0, 0])[None, :] * (1 + p)
    pages = [7, 3, 11, 0, 5, 8, 1, 9, 2, 10]  # logical page i -> physical page
    k[pages[2], 0] = q[0, 0] * 3.0
    k[pages[6], 0] = q[0, 0] * 2.0
    kmin, kmax = qm.page_summaries(k, [0, 10], pages, [P], P)
    sel = qm.quest_selection(q, kmin, kmax, [0, 1], [0, 10], pages, 1, 1, 3)
    assert list(sel[0][0]) == [2, 6, 9], sel
    # the last page scoring best is kept once, at the end, and two others join it
    k[pages[9], 0] = q[0, 0] * 5.0
    kmin, kmax = qm.page_summaries(k, [0, 10], pages, [P], P)
    sel = qm.quest_selection(q, kmin, kmax, [0, 1], [0, 10], pages, 1, 1, 3)
    assert list(sel[0][0]) == [2, 6, 9], sel
    # equal scores (pages 1, 4 and 7 hold the same keys): the earlier pages win
    k[pages[2], 0] = k[pages[0], 0]
    k[pages[6], 0] = k[pages[0], 0]
    for i in (1, 4, 7):
        k[pages[i], 0] = q[0, 0] * 2.0
    kmin, kmax = qm.page_summaries(k, [0, 10], pages, [P], P)
    sel = qm.quest_selection(q, kmin, kmax, [0, 1], [0, 10], pages, 1, 1, 3)
    assert list(sel[0][0]) == [1, 4, 9], sel


def pin_full_budget_is_plain_attention(qm):
    from oracle import attention as att

    kv, P, h_qo, h_kv, d = [45, 16, 3, 70], 8, 4, 2, 8
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(34, kv, P, h_qo, h_kv, d)
    o, lse, sel = qm.quest_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, 0.3, 64)
    ro, rl = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, 0.3)
    assert np.array_equal(o, ro) and np.array_equal(lse, rl)


def pin_kept_keys_brute_force(qm):
    kv, P, h_qo, h_kv, d, budget = [90, 33, 12], 4, 2, 1, 4, 5
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(35, kv, P, h_qo, h_kv, d)
    scale, cap = 0.5, 2.0
    o, lse, sel = qm.quest_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, scale, budget,
                                     cap=cap)
    for r in range(len(kv)):
        for h in range(h_qo):
            keys, vals = [], []
            for i in sel[r][0]:
                kk = _page_keys(k, kv_indptr, kv_indices, last, P, r, int(i))[0]
                vv = _page_keys(v, kv_indptr, kv_indices, last, P, r, int(i))[0]
                keys += list(kk)
                vals += list(vv)
            logits = [cap * math.tanh(scale * sum(float(a) * float(b) for a, b in zip(q[r, h], key)) / cap)
                      for key in keys]
            mx = max(logits)
            z = sum(math.exp(x - mx) for x in logits)
            assert abs(lse[r, h] - (mx + math.log(z))) < 1e-12
            want = [sum(math.exp(x - mx) * float(val[c]) for x, val in zip(logits, vals)) / z for c in range(d)]
            assert np.allclose(o[r, h], want, rtol=0, atol=1e-12)


ALL_QUEST_PINS = [
    pin_summaries_bound_their_keys,
    pin_score_bounds_every_key_and_is_exact_for_one_key,
    pin_kept_pages_are_a_valid_top_set,
    pin_crafted_best_pages,
    pin_full_budget_is_plain_attention,
    pin_kept_keys_brute_force,
]
