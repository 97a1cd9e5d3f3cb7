"""Plain float64 CPU oracle for attention over a block-sparse-row (paged) KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  The library never
calls it, shares no code with it, and this module imports nothing from the
library.

Sources (the FlashInfer explainer page on zenmind.me, "FlashInfer：面向 LLM 推理
服务的高效可定制注意力引擎", which restates the MLSys 2025 paper):
  * Terms, "BSR" and Core mechanism 1 (paper section 3.1.1, Figure 2): the KV cache
    is a block-sparse-row matrix whose non-zero blocks are the physical pages a
    request reads; any (Br, Bc) is allowed.
  * Terms, "ragged tensor": queries and outputs of all requests are packed without
    padding and addressed by one indptr array.
  * Terms, "Attention State and ⊕" (paper section 2.2): the canonical result is the
    pair (O, LSE) and ⊕ combines two such states; it is associative and commutative.
  * Terms, "composable formats" and Core mechanism 2 (paper section 3.1.2, Figure 3):
    several BSR sub-matrices over the same KV pool; only index arrays differ.
  * Terms, "GQA head-group fusion" and Background (paper section 2.1): g = H_qo / H_kv
    query heads share one KV head.
  * Background, challenge 2 (paper section 1): logits soft-cap as a custom score.
  * Section "Reproduction" (paper section 4.2): prefill is run with a causal mask.
  * Background, "variants" (paper sections 1 and 3.2.3): masks such as a sliding
    window and ALiBi are variant axes (the LogitsMask and LogitsTransform
    functors); Quick read item 1 names custom masks for speculative decoding.

What this oracle computes is the plain definition of attention, with no tiling,
online softmax, chunking or plan:

    S = scale * Q K^T ;  S <- cap * tanh(S / cap)  (if cap > 0) ;  causal mask ;
    LSE = log(sum_j exp(S_j)) ;  O = softmax(S) V

Readings where the pages are silent (each is listed in the design notes):
  * LSE uses the natural logarithm.
  * The soft-cap is applied to the scaled logit, before masking; LSE is taken over
    the capped logits.
  * Causal masking is aligned bottom-right: query token t (0-based among the l_qo
    new tokens of its request) sees keys j <= l_kv - l_qo + t.
  * A sliding window of W keys (W >= 1; 0 is no window) uses the same alignment:
    query token t sees keys j > l_kv - l_qo + t - W, that is the W keys ending at
    its own position when the mask is also causal.  The window bounds keys from
    below only; the causal flag bounds them from above.
  * ALiBi (the pages name it, do not define it): query head h has a slope m_h
    (given by the caller) and its logit for key j gains m_h * (j - p), where p is
    the query's bottom-right aligned position l_kv - l_qo + t.  The bias is added to
    the scaled logit, before the soft-cap and the masks.
  * Tree masks for speculative decoding (named, not defined): the l_qo new tokens
    of a request are its last l_qo keys; a boolean matrix M [l_qo, l_qo] per
    request lets token t see key l_kv - l_qo + u iff M[t, u]; keys before the new
    tokens stay visible.  The tree mask applies on top of the causal and window
    masks.
  * Query head h reads KV head floor(h / g).
  * A request with n pages holds l_kv = (n - 1) * P + last_page_len tokens; a
    request with no pages, and a row whose every key is masked, give O = 0 and
    LSE = -inf.
  * The pool is laid out [num_pages, H_kv, P, D] (K and V in separate pools).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "gather_request_kv",
    "attention_dense",
    "bsr_attention",
    "merge_state",
    "merge_states",
    "composable_attention",
    "kv_lengths",
]


def kv_lengths(kv_indptr, last_page_len, page_size):
    """Tokens held by each block row.

    Follows the page-table view of Core mechanism 1: a request owns the pages
    kv_indices[kv_indptr[r]:kv_indptr[r+1]] in logical order; every page but the
    last is full and the last holds last_page_len[r] valid slots.
    """
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    last = np.asarray(last_page_len, dtype=np.int64)
    n_pages = kv_indptr[1:] - kv_indptr[:-1]
    return np.where(n_pages > 0, (n_pages - 1) * page_size + last, 0)


def gather_request_kv(pool, kv_indptr, kv_indices, last_page_len, r, page_size):
    """Logical KV rows of block row r, in token order, as float64 [l_kv, H_kv, D].

    Core mechanism 1 (paper section 3.1.1): the non-zero blocks of block row r are
    the pages it reads; token tau lives in page kv_indices[kv_indptr[r] + tau // P]
    at slot tau % P.  The pool is [num_pages, H_kv, P, D].
    """
    begin, end = int(kv_indptr[r]), int(kv_indptr[r + 1])
    n_pages = end - begin
    if n_pages == 0:
        return np.zeros((0, pool.shape[1], pool.shape[3]), dtype=np.float64)
    l_kv = (n_pages - 1) * page_size + int(last_page_len[r])
    tau = np.arange(l_kv)
    pages = np.asarray(kv_indices[begin:end], dtype=np.int64)[tau // page_size]
    # advanced indices on axes 0 and 2 around a slice: result is [l_kv, H_kv, D]
    return np.asarray(pool[pages, :, tau % page_size, :], dtype=np.float64)


def attention_dense(q, k, v, scale, cap=0.0, visible=None, lowest=None, bias=None, allowed=None):
    """Attention state (O, LSE) of query rows q against keys k and values v.

    q: [n, D], k and v: [L, D] (float64).  visible: None (every key visible) or an
    int array [n] giving, per query row, the largest visible key index (keys
    j > visible[i] are masked); lowest: None or an int array [n] giving the
    smallest visible key index (keys j < lowest[i] are masked); bias: None or an
    [n, L] array added to the scaled logits before the cap (ALiBi); allowed: None
    or a boolean [n, L] array, False masks the key (tree masks).  Returns O [n, D]
    and LSE [n] (natural log).

    The state definition is the one of Terms, "Attention State and ⊕" (paper
    section 2.2); the cap is the soft-cap of Background, challenge 2.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    length = k.shape[0]
    out = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full((n,), -np.inf, dtype=np.float64)
    if n == 0 or length == 0:
        return out, lse
    s = scale * (q @ k.T)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)
    if cap > 0.0:
        s = cap * np.tanh(s / cap)
    if visible is not None:
        cols = np.arange(length)[None, :]
        s = np.where(cols <= np.asarray(visible)[:, None], s, -np.inf)
    if lowest is not None:
        cols = np.arange(length)[None, :]
        s = np.where(cols >= np.asarray(lowest)[:, None], s, -np.inf)
    if allowed is not None:
        s = np.where(np.asarray(allowed, dtype=bool), s, -np.inf)
    m = np.max(s, axis=1)
    live = np.isfinite(m)
    if not np.any(live):
        return out, lse
    s_live = s[live]
    m_live = m[live]
    w = np.exp(s_live - m_live[:, None])
    z = np.sum(w, axis=1)
    out[live] = (w @ v) / z[:, None]
    lse[live] = m_live + np.log(z)
    return out, lse


def bsr_attention(
    q,
    k_pool,
    v_pool,
    qo_indptr,
    kv_indptr,
    kv_indices,
    last_page_len,
    page_size,
    num_qo_heads,
    num_kv_heads,
    scale,
    causal=False,
    cap=0.0,
    window=0,
    alibi_slopes=None,
    tree_masks=None,
):
    """Attention of ragged queries over a BSR/paged KV cache.

    q: [sum l_qo, H_qo, D]; pools: [num_pages, H_kv, P, D].  Returns O
    [sum l_qo, H_qo, D] and LSE [sum l_qo, H_qo], both float64.

    Ragged packing follows Terms, "ragged tensor"; the page gather follows Core
    mechanism 1; the GQA mapping follows Terms, "GQA head-group fusion"; the causal
    mask is the prefill mask of section "Reproduction" (paper section 4.2), aligned
    bottom-right as stated in the module notes; window > 0 adds the sliding-window
    mask of the module notes.  alibi_slopes ([H_qo] or None) adds the ALiBi bias
    and tree_masks (per request a boolean [l_qo, l_qo] array, or None) the tree
    mask of the module notes (Background, variants; paper section 3.2.3).
    """
    q = np.asarray(q)
    total, h_qo, d = q.shape
    assert h_qo == num_qo_heads and num_qo_heads % num_kv_heads == 0
    g = num_qo_heads // num_kv_heads
    out = np.zeros((total, h_qo, v_pool.shape[3]), dtype=np.float64)
    lse = np.full((total, h_qo), -np.inf, dtype=np.float64)
    batch = len(qo_indptr) - 1
    for r in range(batch):
        q0, q1 = int(qo_indptr[r]), int(qo_indptr[r + 1])
        l_qo = q1 - q0
        if l_qo == 0:
            continue
        k_r = gather_request_kv(k_pool, kv_indptr, kv_indices, last_page_len, r, page_size)
        v_r = gather_request_kv(v_pool, kv_indptr, kv_indices, last_page_len, r, page_size)
        l_kv = k_r.shape[0]
        visible = None
        if causal:
            visible = l_kv - l_qo + np.arange(l_qo)
        lowest = None
        if window > 0:
            lowest = l_kv - l_qo + np.arange(l_qo) - window + 1
        allowed = None
        if tree_masks is not None and tree_masks[r] is not None:
            tree = np.asarray(tree_masks[r], dtype=bool)
            assert tree.shape == (l_qo, l_qo) and l_kv >= l_qo, "a tree mask covers the request's new tokens"
            allowed = np.ones((l_qo, l_kv), dtype=bool)
            allowed[:, l_kv - l_qo :] = tree
        positions = l_kv - l_qo + np.arange(l_qo)  # bottom-right aligned query positions
        for h in range(h_qo):
            hk = h // g
            bias = None
            if alibi_slopes is not None:
                bias = float(alibi_slopes[h]) * (np.arange(l_kv)[None, :] - positions[:, None])
            o_h, lse_h = attention_dense(
                np.asarray(q[q0:q1, h, :], dtype=np.float64),
                k_r[:, hk, :],
                v_r[:, hk, :],
                scale,
                cap,
                visible,
                lowest,
                bias,
                allowed,
            )
            out[q0:q1, h, :] = o_h
            lse[q0:q1, h] = lse_h
    return out, lse


def merge_state(o_a, lse_a, o_b, lse_b):
    """The ⊕ of two attention states (Terms, "Attention State and ⊕", paper section 2.2).

    A state (O, LSE) is a softmax-weighted mean O over a key set together with the
    log of that key set's total weight.  Combining two disjoint key sets weights
    each mean by its set's total weight:
        LSE = log(exp(lse_a) + exp(lse_b)),
        O   = (exp(lse_a) O_a + exp(lse_b) O_b) / exp(LSE),
    evaluated with the larger LSE factored out.  (0, -inf) is the identity (the
    empty key set); two empty states give (0, -inf).
    Shapes: o_* [..., D], lse_* [...].
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w_a = np.where(np.isfinite(lse_a), np.exp(lse_a - m_safe), 0.0)
    w_b = np.where(np.isfinite(lse_b), np.exp(lse_b - m_safe), 0.0)
    z = w_a + w_b
    z_safe = np.where(empty, 1.0, z)
    o = (w_a[..., None] * o_a + w_b[..., None] * o_b) / z_safe[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, m_safe + np.log(z_safe))
    return o, lse


def merge_states(states):
    """Left fold of ⊕ over a sequence of (O, LSE) states, in the given order."""
    it = iter(states)
    o, lse = next(it)
    for o_b, lse_b in it:
        o, lse = merge_state(o, lse, o_b, lse_b)
    return o, lse


def composable_attention(
    q,
    k_pool,
    v_pool,
    formats,
    kv_indices,
    page_size,
    num_qo_heads,
    num_kv_heads,
    scale,
    cap=0.0,
):
    """Attention when the KV matrix is split into several BSR sub-matrices.

    Terms, "composable formats" and Core mechanism 2 (paper section 3.1.2,
    Figure 3): each format is a BSR matrix over the same pool, described only by
    index arrays.  Block row b of format f covers query tokens
    [qo_indptr[b], qo_indptr[b+1]) and reads its own pages.  A query token's key
    set is the union of the key sets of the block rows that cover it, taken in
    format order; attention over that union is the result.

    formats: sequence of dicts with keys qo_indptr, kv_indptr, last_page_len and
    kv_indices_offset (offset of the format's indices inside kv_indices).
    Causal masking is not defined for composed formats here.
    """
    q = np.asarray(q)
    total, h_qo, d = q.shape
    g = num_qo_heads // num_kv_heads
    per_token = [[] for _ in range(total)]
    for f in formats:
        qo_indptr = f["qo_indptr"]
        kv_indptr = np.asarray(f["kv_indptr"], dtype=np.int64) + int(f["kv_indices_offset"])
        for b in range(len(qo_indptr) - 1):
            for t in range(int(qo_indptr[b]), int(qo_indptr[b + 1])):
                per_token[t].append((kv_indptr, f["last_page_len"], b))
    out = np.zeros((total, h_qo, v_pool.shape[3]), dtype=np.float64)
    lse = np.full((total, h_qo), -np.inf, dtype=np.float64)
    cache = {}
    for t in range(total):
        key = tuple((id(ip), b) for ip, _, b in per_token[t])
        if key not in cache:
            ks, vs = [], []
            for ip, last, b in per_token[t]:
                ks.append(gather_request_kv(k_pool, ip, kv_indices, last, b, page_size))
                vs.append(gather_request_kv(v_pool, ip, kv_indices, last, b, page_size))
            if ks:
                cache[key] = (np.concatenate(ks, axis=0), np.concatenate(vs, axis=0))
            else:
                cache[key] = (
                    np.zeros((0, k_pool.shape[1], k_pool.shape[3])),
                    np.zeros((0, v_pool.shape[1], v_pool.shape[3])),
                )
        k_t, v_t = cache[key]
        for h in range(h_qo):
            hk = h // g
            o_h, lse_h = attention_dense(
                np.asarray(q[t : t + 1, h, :], dtype=np.float64), k_t[:, hk, :], v_t[:, hk, :], scale, cap
            )
            out[t, h, :] = o_h[0]
            lse[t, h] = lse_h[0]
    return out, lse


def default_scale(head_dim):
    """1/sqrt(D), the scale the pages' first workload states; used for every workload."""
    return 1.0 / math.sqrt(head_dim)
