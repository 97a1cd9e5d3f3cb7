"""Pins of the oracle's sliding-window mask.

Each pin takes the oracle's attention module and raises on a mismatch.  The values
come from the definition of the mask (a window of W keys ending at the query's
bottom-right aligned position; the FlashInfer explainer page names sliding windows
among the mask variants, Background and paper section 3.2.3), computed here by
independent means: a closed form for W = 1, the no-window result for a window that
covers every key, and per-row brute force with math.exp on tiny inputs.
"""

from __future__ import annotations

import math

import numpy as np


def _case(seed, qo_lens, kv_lens, page_size, h_qo, h_kv, d):
    rng = np.random.default_rng(seed)
    n_pages = [(l + page_size - 1) // page_size for l in kv_lens]
    num_pages = sum(n_pages) + 2
    kv_indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int64)
    kv_indices = rng.permutation(num_pages)[: sum(n_pages)]
    last = np.array([l - (n - 1) * page_size if n else page_size for l, n in zip(kv_lens, n_pages)])
    qo_indptr = np.concatenate([[0], np.cumsum(qo_lens)]).astype(np.int64)
    q = rng.standard_normal((int(qo_indptr[-1]), h_qo, d))
    k = rng.standard_normal((num_pages, h_kv, page_size, d))
    v = rng.standard_normal((num_pages, h_kv, page_size, d))
    return q, k, v, qo_indptr, kv_indptr, kv_indices, last


def _key(pool, kv_indptr, kv_indices, page_size, r, h, j):
    """Row j of request r's KV, head h, read straight from the page table."""
    return pool[kv_indices[kv_indptr[r] + j // page_size], h, j % page_size]


def pin_window_one_is_own_key(att):
    """Causal, W = 1: each query sees only the key at its own position, so O is
    that key's value and LSE its scaled logit."""
    qo, kv, P, h_qo, h_kv, d = [3, 1, 5], [7, 4, 5], 3, 4, 2, 16
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(11, qo, kv, P, h_qo, h_kv, d)
    scale = 0.3
    o, lse = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, scale,
                               causal=True, window=1)
    g = h_qo // h_kv
    for r in range(len(qo)):
        for t in range(qo[r]):
            pos = kv[r] - qo[r] + t
            row = int(qo_indptr[r]) + t
            for h in range(h_qo):
                kk = _key(k, kv_indptr, kv_indices, P, r, h // g, pos)
                vv = _key(v, kv_indptr, kv_indices, P, r, h // g, pos)
                assert np.allclose(o[row, h], vv, rtol=0, atol=1e-12), (r, t, h)
                assert abs(lse[row, h] - scale * float(q[row, h] @ kk)) < 1e-12, (r, t, h)


def pin_window_covering_every_key_is_no_window(att):
    """A window at least l_kv long hides nothing, causal or not."""
    qo, kv, P, h_qo, h_kv, d = [4, 2], [9, 6], 2, 2, 1, 8
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(12, qo, kv, P, h_qo, h_kv, d)
    for causal in (False, True):
        ref = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, 0.5, causal=causal)
        got = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, 0.5, causal=causal,
                                window=max(kv))
        assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1]), causal


def pin_window_brute_force(att):
    """Per row, the softmax over exactly the keys j with pos - W < j (and j <= pos
    when causal), summed term by term with math.exp, soft-cap included."""
    qo, kv, P, h_qo, h_kv, d = [3, 4, 1], [8, 4, 10], 3, 2, 1, 4
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(13, qo, kv, P, h_qo, h_kv, d)
    scale = 0.7
    for causal, window, cap in ((True, 3, 0.0), (False, 2, 0.0), (True, 5, 1.5), (False, 6, 2.0)):
        o, lse = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, scale,
                                   causal=causal, cap=cap, window=window)
        for r in range(len(qo)):
            for t in range(qo[r]):
                pos = kv[r] - qo[r] + t
                keys = [j for j in range(kv[r]) if j > pos - window and (not causal or j <= pos)]
                row = int(qo_indptr[r]) + t
                for h in range(h_qo):
                    logits = []
                    for j in keys:
                        x = scale * sum(float(a) * float(b) for a, b in zip(q[row, h], _key(k, kv_indptr, kv_indices, P, r, 0, j)))
                        logits.append(cap * math.tanh(x / cap) if cap > 0 else x)
                    z = sum(math.exp(x) for x in logits)
                    want_o = [sum(math.exp(x) * float(_key(v, kv_indptr, kv_indices, P, r, 0, j)[c])
                                  for x, j in zip(logits, keys)) / z for c in range(d)]
                    assert abs(lse[row, h] - math.log(z)) < 1e-12, (causal, window, r, t, h)
                    assert np.allclose(o[row, h], want_o, rtol=0, atol=1e-12), (causal, window, r, t, h)


ALL_WINDOW_PINS = [pin_window_one_is_own_key, pin_window_covering_every_key_is_no_window, pin_window_brute_force]
