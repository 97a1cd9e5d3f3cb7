"""Plain CPU oracle for writing new K/V rows into the paged (BSR) KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  The library never
calls it, shares no code with it, and this module imports nothing from the
library.

Source: the FlashInfer explainer page on zenmind.me, Core mechanism 1 (paper
section 3.1.1, Figure 2).  Newly generated K/V rows are first packed like the
queries, addressed by the queries' indptr (ragged, no padding), and are then
written into the block-sparse-row KV cache, whose non-zero blocks are the pages
of each request.

Reading where the page is silent (listed in the design notes): the n_r new
tokens of request r are the last n_r tokens of its KV as the page table
describes it after the write, i.e. new token j goes to logical position
tau = l_kv - n_r + j, which lives in page kv_indices[kv_indptr[r] + tau // P]
at slot tau % P (the same bottom-right alignment as the causal mask).  Requests
with n_r > l_kv have no slot for their first n_r - l_kv new tokens; those rows
are not written.

This is pure indexing: the result is exact and the pools keep their dtype.
"""

from __future__ import annotations

import numpy as np

from .attention import kv_lengths

__all__ = ["append_slots", "append_paged_kv"]


def append_slots(append_indptr, kv_indptr, kv_indices, last_page_len, page_size):
    """For every new row i, its (page, slot), or (-1, -1) when it has none.

    Rows are numbered like the queries: request r owns rows
    append_indptr[r] .. append_indptr[r+1] - 1, in token order.
    """
    append_indptr = np.asarray(append_indptr, dtype=np.int64)
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    l_kv = kv_lengths(kv_indptr, last_page_len, page_size)
    total = int(append_indptr[-1])
    page = np.full(total, -1, dtype=np.int64)
    slot = np.full(total, -1, dtype=np.int64)
    for r in range(len(append_indptr) - 1):
        n_r = int(append_indptr[r + 1] - append_indptr[r])
        for j in range(n_r):
            tau = int(l_kv[r]) - n_r + j
            if tau < 0:
                continue
            page[append_indptr[r] + j] = kv_indices[kv_indptr[r] + tau // page_size]
            slot[append_indptr[r] + j] = tau % page_size
    return page, slot


def append_paged_kv(k_pool, v_pool, k_new, v_new, append_indptr, kv_indptr, kv_indices, last_page_len,
                    page_size):
    """Copies of the pools [num_pages, H_kv, P, D] with the new rows written.

    k_new, v_new: [total_new, H_kv, D], rows packed by append_indptr.  Every head
    of a new token goes to the same (page, slot) of its own head plane.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    page, slot = append_slots(append_indptr, kv_indptr, kv_indices, last_page_len, page_size)
    for i in range(len(page)):
        if page[i] < 0:
            continue
        k_out[page[i], :, slot[i], :] = k_new[i]
        v_out[page[i], :, slot[i], :] = v_new[i]
    return k_out, v_out
