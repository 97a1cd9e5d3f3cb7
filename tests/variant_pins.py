"""Pins of the oracle's ALiBi bias and tree masks (the variant functors the
FlashInfer explainer page names in Background, challenge 2, and paper section
3.2.3; Quick read item 1 names custom masks for speculative decoding).

Each pin takes the oracle's attention module and raises on a mismatch.  The values
come from independent means: closed forms of a two-key example (stored with their
derivations in tests/golden/variant_closed_forms.json), the softmax's invariance
under a per-row shift of the logits, the causal mask as a special tree, a zero
query whose weights are a geometric sequence, and per-row brute force with
math.exp over an explicit list of visible keys.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "variant_closed_forms.json")


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
    return pool[kv_indices[kv_indptr[r] + j // page_size], h, j % page_size]


def random_tree(rng, n):
    """A speculative-decoding token tree over n draft tokens: token t's parent is
    an earlier token (or none); t sees itself and its ancestors."""
    parent = [-1] + [int(rng.integers(-1, t)) for t in range(1, n)]
    m = np.zeros((n, n), dtype=bool)
    for t in range(n):
        u = t
        while u >= 0:
            m[t, u] = True
            u = parent[u]
    return m


def _brute(att, q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, kv, qo, scale, causal, cap, window,
           slopes, trees):
    """Compare the oracle with a term-by-term softmax over each row's visible keys."""
    o, lse = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, scale, causal=causal,
                               cap=cap, window=window, alibi_slopes=slopes, tree_masks=trees)
    g = h_qo // h_kv
    d = q.shape[2]
    for r in range(len(qo)):
        for t in range(qo[r]):
            pos = kv[r] - qo[r] + t
            row = int(qo_indptr[r]) + t
            keys = []
            for j in range(kv[r]):
                if causal and j > pos:
                    continue
                if window > 0 and j <= pos - window:
                    continue
                u = j - (kv[r] - qo[r])
                if trees is not None and trees[r] is not None and u >= 0 and not trees[r][t][u]:
                    continue
                keys.append(j)
            for h in range(h_qo):
                hk = h // g
                logits = []
                for j in keys:
                    x = scale * sum(float(a) * float(b) for a, b in zip(q[row, h], _key(k, kv_indptr, kv_indices, P, r, hk, j)))
                    if slopes is not None:
                        x += float(slopes[h]) * (j - pos)
                    logits.append(cap * math.tanh(x / cap) if cap > 0 else x)
                if not keys:
                    assert lse[row, h] == -math.inf and not np.any(o[row, h]), (r, t, h)
                    continue
                mx = max(logits)
                z = sum(math.exp(x - mx) for x in logits)
                want_o = [sum(math.exp(x - mx) * float(_key(v, kv_indptr, kv_indices, P, r, hk, j)[c])
                              for x, j in zip(logits, keys)) / z for c in range(d)]
                assert abs(lse[row, h] - (mx + math.log(z))) < 1e-11, (r, t, h)
                assert np.allclose(o[row, h], want_o, rtol=0, atol=1e-12), (r, t, h)


def pin_alibi_closed_forms(att):
    """One query (position 1) over k0 = (1, 0), k1 = (0, 1) with values e0, e1, scale
    1: the logits are (1 - m, 0), so O = (sigmoid(1 - m), sigmoid(m - 1)) and
    LSE = log(exp(1 - m) + 1); with a cap c the logits are c tanh((1 - m) / c), 0."""
    with open(GOLDEN) as f:
        cases = [c for c in json.load(f)["cases"] if c["kind"] == "alibi"]
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    for c in cases:
        o, lse = att.bsr_attention(q, k, v, [0, 1], [0, 1], [0], [2], 2, 1, 1, 1.0, cap=c["cap"],
                                   alibi_slopes=[c["slope"]])
        assert abs(lse[0, 0] - c["lse"]) < 1e-14, c
        assert abs(o[0, 0, 0] - c["o"][0]) < 1e-14 and abs(o[0, 0, 1] - c["o"][1]) < 1e-14, c


def pin_alibi_zero_slope_is_plain(att):
    qo, kv, P, h_qo, h_kv, d = [3, 1], [7, 40], 3, 4, 2, 8
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(21, qo, kv, P, h_qo, h_kv, d)
    ref = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, 0.4, causal=True, cap=3.0)
    got = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, 0.4, causal=True, cap=3.0,
                            alibi_slopes=[0.0] * h_qo)
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


def pin_alibi_is_a_row_shift_of_a_key_ramp(att):
    """Without a cap, the bias m (j - p) is the ramp m j shifted by the row constant
    -m p: the softmax (O) is the ramp's, and LSE is the ramp's minus m p.  This
    fixes the bottom-right position p = l_kv - l_qo + t of every row."""
    qo, kv, P, h_qo, h_kv, d = [4, 1], [9, 30], 4, 2, 1, 8
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(22, qo, kv, P, h_qo, h_kv, d)
    slopes = [0.25, -0.5]
    o, lse = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, 0.5, causal=True,
                               alibi_slopes=slopes)
    for r in range(len(qo)):
        kr = att.gather_request_kv(k, kv_indptr, kv_indices, last, r, P)
        vr = att.gather_request_kv(v, kv_indptr, kv_indices, last, r, P)
        q0 = int(qo_indptr[r])
        for h in range(h_qo):
            for t in range(qo[r]):
                pos = kv[r] - qo[r] + t
                ramp = slopes[h] * np.arange(kv[r])[None, :]
                o2, l2 = att.attention_dense(q[q0 + t : q0 + t + 1, h], kr[:, 0], vr[:, 0], 0.5,
                                             visible=np.array([pos]), bias=ramp)
                assert np.allclose(o[q0 + t, h], o2[0], rtol=0, atol=1e-12), (r, h, t)
                assert abs(lse[q0 + t, h] - (l2[0] - slopes[h] * pos)) < 1e-12, (r, h, t)


def pin_alibi_zero_query_is_geometric(att):
    """Q = 0, no cap: the weights over keys 0..L-1 are exp(m (j - p)), a geometric
    sequence, so LSE = -m p + log((exp(m L) - 1) / (exp(m) - 1))."""
    kv, P, d = [12, 5], 4, 4
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(23, [1, 1], kv, P, 2, 2, d)
    q = np.zeros_like(q)
    slopes = [0.3, -0.7]
    o, lse = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, 2, 2, 1.0, alibi_slopes=slopes)
    for r, L in enumerate(kv):
        p = L - 1
        for h, m in enumerate(slopes):
            want = -m * p + math.log((math.exp(m * L) - 1.0) / (math.exp(m) - 1.0))
            assert abs(lse[r, h] - want) < 1e-12, (r, h)


def pin_alibi_brute_force(att):
    qo, kv, P, h_qo, h_kv, d = [3, 2, 1], [8, 5, 11], 3, 4, 2, 4
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(24, qo, kv, P, h_qo, h_kv, d)
    slopes = [0.5, 0.25, -0.125, 1.0]
    for causal, cap, window in ((True, 0.0, 0), (False, 0.0, 0), (True, 2.5, 0), (False, 1.5, 4), (True, 0.0, 3)):
        _brute(att, q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, kv, qo, 0.6, causal, cap, window,
               slopes, None)


def pin_tree_all_true_is_unmasked(att):
    qo, kv, P, h_qo, h_kv, d = [3, 4], [7, 9], 2, 2, 1, 8
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(25, qo, kv, P, h_qo, h_kv, d)
    ref = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, 0.5)
    trees = [np.ones((n, n), dtype=bool) for n in qo]
    got = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, 0.5, tree_masks=trees)
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


def pin_tree_chain_is_causal(att):
    """The chain tree (each draft token's ancestors are all earlier ones) is the
    bottom-right causal mask."""
    qo, kv, P, h_qo, h_kv, d = [3, 5, 1], [7, 9, 4], 3, 4, 2, 8
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(26, qo, kv, P, h_qo, h_kv, d)
    ref = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, 0.5, causal=True)
    trees = [np.tril(np.ones((n, n), dtype=bool)) for n in qo]
    got = att.bsr_attention(q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, 0.5, tree_masks=trees)
    assert np.allclose(ref[0], got[0], rtol=0, atol=1e-15) and np.array_equal(ref[1], got[1])


def pin_tree_brute_force(att):
    qo, kv, P, h_qo, h_kv, d = [5, 1, 4, 6], [9, 6, 4, 6], 3, 4, 2, 4
    q, k, v, qo_indptr, kv_indptr, kv_indices, last = _case(27, qo, kv, P, h_qo, h_kv, d)
    rng = np.random.default_rng(28)
    trees = [random_tree(rng, n) for n in qo]
    trees[1] = None  # a request without a tree
    for causal, cap, slopes in ((True, 0.0, None), (False, 0.0, None), (True, 2.0, None),
                                (True, 0.0, [0.5, -0.25, 0.125, 1.0])):
        _brute(att, q, k, v, qo_indptr, kv_indptr, kv_indices, last, P, h_qo, h_kv, kv, qo, 0.6, causal, cap, 0,
               slopes, trees)


ALL_VARIANT_PINS = [
    pin_alibi_closed_forms,
    pin_alibi_zero_slope_is_plain,
    pin_alibi_is_a_row_shift_of_a_key_ramp,
    pin_alibi_zero_query_is_geometric,
    pin_alibi_brute_force,
    pin_tree_all_true_is_unmasked,
    pin_tree_chain_is_causal,
    pin_tree_brute_force,
]
