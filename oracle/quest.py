"""Plain CPU oracle for Quest-style page-budget sparse decode over the BSR cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  The library never
calls it, shares no code with it, and this module imports nothing from the
library.

Source: the FlashInfer explainer page on zenmind.me, Applicable scenarios item 5
(paper Appendix G.5, Tables 9-11): long-context KV-pruning algorithms of the
Quest kind keep a budget of KV pages per step and run the block-sparse attention
(pages of 16 keys) over the kept pages only; the page quotes a sequence of 32768
keys, a budget of 64 pages, 32 query and 32 KV heads, head dim 128.  The kept
pages are a BSR matrix like any other: only the page list changes.

The pages name the method but not its page choice.  Readings (Quest's published
criterion, restated; each is listed in the design notes):
  * every page keeps, per KV head, the elementwise minimum and maximum of its
    valid keys (the last page of a request holds last_page_len of them);
  * a query head's score of a page is sum_d max(q_d * min_d, q_d * max_d), an
    upper bound of q.k over the page's keys;
  * with grouped heads, a KV head's score of a page is the largest score of its g
    query heads (a page any of them may need is kept);
  * per request and KV head, the page holding the newest keys (the last page) is
    always kept; the other budget - 1 places go to the other pages with the
    highest scores, ties to the earlier page; with at most `budget` pages every
    page is kept;
  * the kept pages are listed in logical order (the last page last), and the
    result is plain attention (the definition in attention.py) over exactly the
    kept keys.
Decode only: each request has one query token.  Scores are computed in float64.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_dense

__all__ = ["page_summaries", "page_scores", "select_pages", "quest_selection", "quest_attention"]


def page_summaries(k_pool, kv_indptr, kv_indices, last_page_len, page_size):
    """Elementwise min and max of each referenced page's valid keys, per KV head.

    Returns kmin, kmax float64 [num_pages, H_kv, D]; pages no request references
    are NaN.
    """
    k_pool = np.asarray(k_pool)
    num_pages, h_kv, _, d = k_pool.shape
    kmin = np.full((num_pages, h_kv, d), np.nan)
    kmax = np.full((num_pages, h_kv, d), np.nan)
    for r in range(len(kv_indptr) - 1):
        b, e = int(kv_indptr[r]), int(kv_indptr[r + 1])
        for i in range(b, e):
            page = int(kv_indices[i])
            valid = page_size if i < e - 1 else int(last_page_len[r])
            keys = np.asarray(k_pool[page, :, :valid, :], dtype=np.float64)  # [H_kv, valid, D]
            kmin[page] = keys.min(axis=1)
            kmax[page] = keys.max(axis=1)
    return kmin, kmax


def page_scores(q_tok, kmin_pages, kmax_pages, group):
    """Scores of n pages for each KV head: [H_kv, n].

    q_tok: [H_qo, D] (one query token); kmin_pages, kmax_pages: [n, H_kv, D].
    Query head h scores a page with sum_d max(q_d min_d, q_d max_d); a KV head
    takes the maximum over its group of query heads.
    """
    q_tok = np.asarray(q_tok, dtype=np.float64)
    h_qo = q_tok.shape[0]
    h_kv = h_qo // group
    n = kmin_pages.shape[0]
    out = np.full((h_kv, n), -np.inf)
    for h in range(h_qo):
        hk = h // group
        qh = q_tok[h][None, :]
        ub = np.sum(np.maximum(qh * kmin_pages[:, hk, :], qh * kmax_pages[:, hk, :]), axis=1)
        out[hk] = np.maximum(out[hk], ub)
    return out


def select_pages(scores, budget):
    """Logical positions of the kept pages of one request and KV head.

    scores: [n] (the last entry is the last page).  The last page is always kept;
    the budget - 1 best of the others (ties to the earlier page) join it.  Returned
    in ascending order, so the last page comes last.
    """
    n = len(scores)
    if n <= budget:
        return np.arange(n)
    others = sorted(range(n - 1), key=lambda i: (-float(scores[i]), i))[: budget - 1]
    return np.array(sorted(others) + [n - 1])


def quest_selection(q, kmin, kmax, qo_indptr, kv_indptr, kv_indices, num_qo_heads, num_kv_heads, budget):
    """Kept page positions (logical, within the request) per request and KV head:
    a list over requests of lists over KV heads."""
    g = num_qo_heads // num_kv_heads
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    out = []
    for r in range(len(kv_indptr) - 1):
        b, e = int(kv_indptr[r]), int(kv_indptr[r + 1])
        assert int(qo_indptr[r + 1]) - int(qo_indptr[r]) == 1, "decode: one query token per request"
        t = int(qo_indptr[r])
        ids = kv_indices[b:e]
        sc = page_scores(q[t], kmin[ids], kmax[ids], g)
        out.append([select_pages(sc[h], budget) for h in range(num_kv_heads)])
    return out


def quest_attention(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, last_page_len, page_size, num_qo_heads,
                    num_kv_heads, scale, budget, cap=0.0):
    """Quest-style decode: summaries, scores, kept pages, then plain attention over
    the kept keys.  Returns O [B, H_qo, D], LSE [B, H_qo] (float64) and the kept
    page positions per request and KV head."""
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    kmin, kmax = page_summaries(k_pool, kv_indptr, kv_indices, last_page_len, page_size)
    sel = quest_selection(q, kmin, kmax, qo_indptr, kv_indptr, kv_indices, num_qo_heads, num_kv_heads, budget)
    g = num_qo_heads // num_kv_heads
    total, h_qo, d = np.asarray(q).shape
    out = np.zeros((total, h_qo, v_pool.shape[3]))
    lse = np.full((total, h_qo), -np.inf)
    for r in range(len(kv_indptr) - 1):
        b, e = int(kv_indptr[r]), int(kv_indptr[r + 1])
        t = int(qo_indptr[r])
        for hk in range(num_kv_heads):
            keys, vals = [], []
            for pos in sel[r][hk]:
                page = int(kv_indices[b + pos])
                valid = page_size if b + pos < e - 1 else int(last_page_len[r])
                keys.append(np.asarray(k_pool[page, hk, :valid, :], dtype=np.float64))
                vals.append(np.asarray(v_pool[page, hk, :valid, :], dtype=np.float64))
            kk = np.concatenate(keys) if keys else np.zeros((0, d))
            vv = np.concatenate(vals) if vals else np.zeros((0, v_pool.shape[3]))
            for j in range(g):
                h = hk * g + j
                o1, l1 = attention_dense(np.asarray(q[t : t + 1, h, :], dtype=np.float64), kk, vv, scale, cap)
                out[t, h] = o1[0]
                lse[t, h] = l1[0]
    return out, lse, sel
