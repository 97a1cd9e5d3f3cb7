"""Pins of the K/V append oracle (Core mechanism 1 of the FlashInfer explainer page,
paper section 3.1.1: new K/V rows are packed like the queries, then written into
the BSR cache).  Each pin takes the oracle's append module as an argument so that
planted mistakes can be checked against the same pins.

* a worked example whose slots are derived by hand (page size 3, a new token
  that starts a page, one that ends one);
* requests with more new tokens than KV positions (rows without a slot are not
  written);
* a cache holding the head of each sequence, with the tail appended, equals the
  cache laid out from the whole sequence (pages permuted, P in {1, 2, 3, 16}),
  using this file's own page-table builder;
* every untouched slot keeps its previous contents (NaN stays NaN).
"""

from __future__ import annotations

import numpy as np


def _pools(num_pages, h_kv, page_size, d, fill=np.nan):
    return (np.full((num_pages, h_kv, page_size, d), fill), np.full((num_pages, h_kv, page_size, d), fill))


def pin_append_worked(A):
    # P = 3; request 0 owns pages [5, 2] and holds 5 tokens after the write
    # (last page 2 slots), 2 of them new -> logical positions 3 and 4 -> page 2
    # (kv_indices[0 + 3 // 3]) slots 0 and 1.  Request 1 owns page [0], holds 1
    # token, new -> page 0 slot 0.  Request 2 has no new tokens.
    append_indptr = np.array([0, 2, 3, 3], dtype=np.int32)
    kv_indptr = np.array([0, 2, 3, 4], dtype=np.int32)
    kv_indices = np.array([5, 2, 0, 4], dtype=np.int32)
    last = np.array([2, 1, 3], dtype=np.int32)
    page, slot = A.append_slots(append_indptr, kv_indptr, kv_indices, last, 3)
    assert page.tolist() == [2, 2, 0], page
    assert slot.tolist() == [0, 1, 0], slot
    k_pool, v_pool = _pools(6, 2, 3, 4)
    k_new = np.arange(3 * 2 * 4, dtype=np.float64).reshape(3, 2, 4)
    v_new = -k_new - 1.0
    k_out, v_out = A.append_paged_kv(k_pool, v_pool, k_new, v_new, append_indptr, kv_indptr, kv_indices, last, 3)
    for i, (pg, sl) in enumerate([(2, 0), (2, 1), (0, 0)]):
        assert np.array_equal(k_out[pg, :, sl, :], k_new[i])
        assert np.array_equal(v_out[pg, :, sl, :], v_new[i])
    written = np.zeros(k_pool.shape[:3], dtype=bool)
    written[2, :, 0] = written[2, :, 1] = written[0, :, 0] = True
    assert np.all(np.isnan(k_out[~written])) and np.all(np.isnan(v_out[~written]))
    assert np.all(np.isnan(k_pool)), "the input pool must not be modified"


def pin_append_overflow(A):
    # 4 new tokens for a request that holds 2 (one page of P = 16, last = 2): only
    # the last two rows have positions (0 and 1); the first two are not written.
    append_indptr = np.array([0, 4], dtype=np.int32)
    page, slot = A.append_slots(append_indptr, np.array([0, 1]), np.array([3]), np.array([2]), 16)
    assert page.tolist() == [-1, -1, 3, 3] and slot.tolist() == [-1, -1, 0, 1]
    # a request without pages has no slot at all
    page, slot = A.append_slots(np.array([0, 1]), np.array([0, 0]), np.array([], dtype=np.int32), np.array([16]), 16)
    assert page.tolist() == [-1]


def _layout(seqs, page_size, order, num_pages, lens=None):
    """Pool [num_pages, H, P, D] holding each sequence in pages order[...], NaN elsewhere.

    Pages are allotted for lens (default: the sequences' own lengths), so a prefix of
    each sequence can be laid out in the pages of the whole sequence."""
    h, d = seqs[0].shape[1], seqs[0].shape[2]
    lens = [s.shape[0] for s in seqs] if lens is None else lens
    pool = np.full((num_pages, h, page_size, d), np.nan)
    kv_indptr, kv_indices, last = [0], [], []
    nxt = 0
    for s, l in zip(seqs, lens):
        n = (l + page_size - 1) // page_size
        pages = order[nxt : nxt + n]
        nxt += n
        for tau in range(s.shape[0]):
            pool[pages[tau // page_size], :, tau % page_size, :] = s[tau]
        kv_indices.extend(int(p) for p in pages)
        kv_indptr.append(kv_indptr[-1] + n)
        last.append(l - (n - 1) * page_size if n > 0 else page_size)
    return pool, np.array(kv_indptr), np.array(kv_indices), np.array(last)


def pin_append_completes_layout(A):
    rng = np.random.default_rng(11)
    for page_size in (1, 2, 3, 16):
        lens = [1, 7, 16, 33, 40]
        new = [1, 3, 16, 1, 40]  # a decode token, a few, a whole page, a prefill
        k_full = [rng.standard_normal((l, 2, 8)) for l in lens]
        v_full = [rng.standard_normal((l, 2, 8)) for l in lens]
        need = sum((l + page_size - 1) // page_size for l in lens)
        num_pages = need + 3
        order = rng.permutation(num_pages)
        k_ref, kv_indptr, kv_indices, last = _layout(k_full, page_size, order, num_pages)
        v_ref, _, _, _ = _layout(v_full, page_size, order, num_pages)
        k_head, _, _, _ = _layout([k[: l - n] for k, l, n in zip(k_full, lens, new)], page_size, order, num_pages, lens)
        v_head, _, _, _ = _layout([v[: l - n] for v, l, n in zip(v_full, lens, new)], page_size, order, num_pages, lens)
        k_new = np.concatenate([k[l - n :] for k, l, n in zip(k_full, lens, new)])
        v_new = np.concatenate([v[l - n :] for v, l, n in zip(v_full, lens, new)])
        append_indptr = np.concatenate([[0], np.cumsum(new)])
        k_out, v_out = A.append_paged_kv(k_head, v_head, k_new, v_new, append_indptr, kv_indptr, kv_indices, last,
                                         page_size)
        assert np.array_equal(k_out, k_ref, equal_nan=True), page_size
        assert np.array_equal(v_out, v_ref, equal_nan=True), page_size


ALL_APPEND_PINS = [pin_append_worked, pin_append_overflow, pin_append_completes_layout]
