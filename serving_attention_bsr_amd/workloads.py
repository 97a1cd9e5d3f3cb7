"""Seeded synthetic inputs for BSR attention: page tables, ragged queries, KV pools.

This module builds inputs only.  It holds none of the attention arithmetic and is
the one module that both the HIP path's tests/benchmark and the CPU oracle are fed
from.  It imports nothing from the rest of the package.

Recipe (every workload):
  * numpy ``Generator(PCG64(seed))`` draws the lengths first, then the physical
    page permutation of the pool;
  * ``torch.Generator().manual_seed(seed)`` draws Q, then the K pool, then the V
    pool, as N(0, 1) float32, then rounds them to the workload dtype (bfloat16 by
    round-to-nearest-even);
  * pool slots that no request references (unused pages and the tail of each last
    page) are set to NaN, so a kernel that reads them into the softmax, or
    multiplies them by a zero probability, produces NaN;
  * lengths "uniform in [a, b]" are integers uniform on the inclusive range.

Layouts: Q and O [sum l_qo, H_qo, D]; K and V pools [num_pages, H_kv, P, D];
index arrays int32.  Pages are shuffled in a pool with 12.5 % spare pages.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}
# bf16 queries and outputs over a K/V cache of OCP FP8 E4M3 codes: K and V are
# drawn like the others and rounded to E4M3 (nearest even) after the unused
# slots are filled with NaN
KV_FP8 = "bf16_kv_fp8"


@dataclasses.dataclass
class Format:
    """One BSR sub-matrix of a composed KV matrix (index arrays only)."""

    qo_indptr: np.ndarray  # [num_block_rows + 1] ranges of query tokens
    kv_indptr: np.ndarray  # [num_block_rows + 1] page ranges (relative to the offset)
    last_page_len: np.ndarray  # [num_block_rows]
    kv_indices_offset: int  # where this format's page ids start in kv_indices

    def as_dict(self):
        return dict(
            qo_indptr=self.qo_indptr,
            kv_indptr=self.kv_indptr,
            last_page_len=self.last_page_len,
            kv_indices_offset=self.kv_indices_offset,
        )


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    causal: bool
    cap: float
    scale: float
    qo_indptr: np.ndarray
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    last_page_len: np.ndarray
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    # composed (multi-format) description of the same KV matrix, if any
    formats: Optional[List[Format]] = None
    # sliding window in keys (0: none)
    window: int = 0
    kv_indices_formats: Optional[np.ndarray] = None

    @property
    def batch(self):
        return len(self.qo_indptr) - 1

    @property
    def qo_lens(self):
        return np.diff(self.qo_indptr.astype(np.int64))

    @property
    def kv_lens(self):
        n = np.diff(self.kv_indptr.astype(np.int64))
        return np.where(n > 0, (n - 1) * self.page_size + self.last_page_len.astype(np.int64), 0)

    @property
    def group(self):
        return self.num_qo_heads // self.num_kv_heads


def _page_table(kv_lens, page_size, perm):
    """Consecutive runs of the permuted pool, one run per request."""
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    n_pages = (kv_lens + page_size - 1) // page_size
    kv_indptr = np.zeros(len(kv_lens) + 1, dtype=np.int64)
    kv_indptr[1:] = np.cumsum(n_pages)
    kv_indices = perm[: kv_indptr[-1]].astype(np.int32)
    last = np.where(n_pages > 0, kv_lens - (n_pages - 1) * page_size, 0)
    # a request with no pages has no last page; store page_size as a placeholder
    last = np.where(n_pages > 0, last, page_size)
    return kv_indptr.astype(np.int32), kv_indices, last.astype(np.int32)


def _pool_pages(needed, spare=0.125):
    return max(1, int(math.ceil(needed * (1.0 + spare))))


def _draw_tensors(seed, total_q, num_pages, h_qo, h_kv, page_size, d, dtype):
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn((total_q, h_qo, d), generator=gen, dtype=torch.float32)
    k = torch.randn((num_pages, h_kv, page_size, d), generator=gen, dtype=torch.float32)
    v = torch.randn((num_pages, h_kv, page_size, d), generator=gen, dtype=torch.float32)
    if dtype == KV_FP8:
        return q.to(torch.bfloat16), k, v  # K, V rounded to E4M3 by the caller, after poisoning
    t = DTYPES[dtype]
    return q.to(t), k.to(t), v.to(t)


def _poison_unused(pool, used_pages, used_slots):
    """NaN-fill every slot that no request references.

    used_pages: page ids in use; used_slots: matching count of valid slots.
    """
    mask = torch.ones(pool.shape[0], pool.shape[2], dtype=torch.bool)
    pages = torch.as_tensor(np.asarray(used_pages, dtype=np.int64))
    slots = torch.as_tensor(np.asarray(used_slots, dtype=np.int64))
    ar = torch.arange(pool.shape[2])
    mask[pages] = ar[None, :] >= slots[:, None]
    pool.masked_fill_(mask[:, None, :, None], float("nan"))


def _used_slots(kv_indptr, kv_indices, last_page_len, page_size):
    pages, slots = [], []
    for r in range(len(kv_indptr) - 1):
        b, e = int(kv_indptr[r]), int(kv_indptr[r + 1])
        for i in range(b, e):
            pages.append(int(kv_indices[i]))
            slots.append(page_size if i < e - 1 else int(last_page_len[r]))
    return pages, slots


def build(
    name,
    seed,
    qo_lens: Sequence[int],
    kv_lens: Sequence[int],
    page_size: int,
    num_qo_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str = "bf16",
    causal: bool = False,
    cap: float = 0.0,
    pool_pages: Optional[int] = None,
    rng: Optional[np.random.Generator] = None,
    poison: bool = True,
    tensors: bool = True,
    window: int = 0,
) -> Workload:
    """A single-format workload from explicit lengths (lengths drawn by the caller).

    tensors=False builds the index arrays only (q, k_pool, v_pool are None).
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    qo_lens = np.asarray(qo_lens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    needed = int(np.sum((kv_lens + page_size - 1) // page_size))
    if pool_pages is None:
        pool_pages = _pool_pages(needed)
    perm = rng.permutation(pool_pages)
    kv_indptr, kv_indices, last = _page_table(kv_lens, page_size, perm)
    qo_indptr = np.zeros(len(qo_lens) + 1, dtype=np.int64)
    qo_indptr[1:] = np.cumsum(qo_lens)
    q = k = v = None
    if tensors:
        q, k, v = _draw_tensors(
            seed, int(qo_indptr[-1]), pool_pages, num_qo_heads, num_kv_heads, page_size, head_dim, dtype
        )
    if tensors and poison:
        pages, slots = _used_slots(kv_indptr, kv_indices, last, page_size)
        _poison_unused(k, pages, slots)
        _poison_unused(v, pages, slots)
    if tensors and dtype == KV_FP8:
        k = k.to(torch.float8_e4m3fn)
        v = v.to(torch.float8_e4m3fn)
    return Workload(
        name=name,
        dtype=dtype,
        num_qo_heads=num_qo_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        page_size=page_size,
        causal=causal,
        cap=cap,
        scale=1.0 / math.sqrt(head_dim),
        qo_indptr=qo_indptr.astype(np.int32),
        kv_indptr=kv_indptr,
        kv_indices=kv_indices,
        last_page_len=last,
        q=q,
        k_pool=k,
        v_pool=v,
        window=window,
    )


# --------------------------------------------------------------------------- #
# The five named workloads.  Their shapes stand in for the pages' serving
# workloads (batch decode, the skewed long-context case of the scheduler
# ablation, causal ragged prefill over a radix-tree cache with one-token pages,
# and parallel generation over a shared prefix).
# --------------------------------------------------------------------------- #

def tiny_decode_f32(seed=1, tensors=True):
    """4 decode requests, KV {17, 64, 100, 255}, P=16, 64-page pool, 8/2 heads, D=64, fp32."""
    return build(
        "tiny_decode_f32", seed, [1, 1, 1, 1], [17, 64, 100, 255], 16, 8, 2, 64,
        dtype="f32", pool_pages=64, tensors=tensors,
    )


def batch_decode(seed=2, batch=64, lo=512, hi=8192, tensors=True):
    """Batch decode, Llama-3-8B attention shape: 32/8 heads, D=128, P=16, bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kv = rng.integers(lo, hi, size=batch, endpoint=True)
    return build("batch_decode", seed, [1] * batch, kv, 16, 32, 8, 128, dtype="bf16", rng=rng, tensors=tensors)


def batch_decode_window(seed=7, batch=64, lo=512, hi=8192, window=4096, tensors=True):
    """Batch decode with a 4096-key sliding window: the batch decode shapes, bf16;
    requests longer than the window read only its last 4096 keys."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kv = rng.integers(lo, hi, size=batch, endpoint=True)
    return build("batch_decode_window", seed, [1] * batch, kv, 16, 32, 8, 128, dtype="bf16", rng=rng,
                 tensors=tensors, window=window)


def batch_decode_fp8(seed=6, batch=64, lo=512, hi=8192, tensors=True):
    """Batch decode with an FP8 (E4M3) K/V cache: the batch decode shapes, bf16 Q/O."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kv = rng.integers(lo, hi, size=batch, endpoint=True)
    return build("batch_decode_fp8", seed, [1] * batch, kv, 16, 32, 8, 128, dtype=KV_FP8, rng=rng, tensors=tensors)


def skewed_long_decode(seed=3, long_len=131072, short_len=1024, n_short=15, cap=30.0, tensors=True):
    """One 131072-token request and 15 of 1024 tokens, soft-cap 30, 32/8 heads, D=128."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kv = [long_len] + [short_len] * n_short
    return build(
        "skewed_long_decode", seed, [1] * len(kv), kv, 16, 32, 8, 128, dtype="bf16", cap=cap, rng=rng,
        tensors=tensors,
    )


def ragged_causal_prefill(seed=4, batch=8, qo_lo=128, qo_hi=4096, pre_lo=0, pre_hi=4096, tensors=True):
    """Causal prefill: l_qo ~ U[128,4096], cached prefix ~ U[0,4096], P=1, 32/8 heads, D=128."""
    rng = np.random.Generator(np.random.PCG64(seed))
    qo = rng.integers(qo_lo, qo_hi, size=batch, endpoint=True)
    prefix = rng.integers(pre_lo, pre_hi, size=batch, endpoint=True)
    return build(
        "ragged_causal_prefill", seed, qo, prefix + qo, 1, 32, 8, 128, dtype="bf16", causal=True, rng=rng,
        tensors=tensors,
    )


def ragged_causal_prefill_fp8(seed=11, batch=8, qo_lo=128, qo_hi=4096, pre_lo=0, pre_hi=4096, tensors=True):
    """The ragged causal prefill shapes (P=1, 32/8 heads, D=128) over an FP8 (E4M3)
    K/V cache with bf16 queries and outputs."""
    rng = np.random.Generator(np.random.PCG64(seed))
    qo = rng.integers(qo_lo, qo_hi, size=batch, endpoint=True)
    prefix = rng.integers(pre_lo, pre_hi, size=batch, endpoint=True)
    return build(
        "ragged_causal_prefill_fp8", seed, qo, prefix + qo, 1, 32, 8, 128, dtype=KV_FP8, causal=True, rng=rng,
        tensors=tensors,
    )


def shared_prefix_composable(
    seed=5, branches=64, prefix_len=8192, suf_lo=64, suf_hi=512, page_size=16,
    num_qo_heads=32, num_kv_heads=8, head_dim=256, dtype="bf16", tensors=True,
):
    """Parallel generation: `branches` decode rows share one prefix, each with its own suffix.

    The KV matrix is described twice over the same pool: as two composed formats
    (the shared prefix as one block row covering every branch, and one block row per
    branch for its suffix), and as one plain format in which every branch lists the
    prefix pages followed by its own.  The prefix is a whole number of pages.
    """
    assert prefix_len % page_size == 0
    rng = np.random.Generator(np.random.PCG64(seed))
    suf = rng.integers(suf_lo, suf_hi, size=branches, endpoint=True)
    n_prefix_pages = prefix_len // page_size
    n_suf_pages = (suf + page_size - 1) // page_size
    needed = n_prefix_pages + int(np.sum(n_suf_pages))
    pool_pages = _pool_pages(needed)
    perm = rng.permutation(pool_pages)
    prefix_pages = perm[:n_prefix_pages].astype(np.int32)
    suf_indptr, suf_indices, suf_last = _page_table(suf, page_size, perm[n_prefix_pages:])
    # plain single-format description: prefix pages then own pages, per branch
    single_indices = []
    single_indptr = [0]
    for b in range(branches):
        single_indices.append(prefix_pages)
        single_indices.append(suf_indices[suf_indptr[b] : suf_indptr[b + 1]])
        single_indptr.append(single_indptr[-1] + n_prefix_pages + int(n_suf_pages[b]))
    single_indices = np.concatenate(single_indices).astype(np.int32)
    qo_indptr = np.arange(branches + 1, dtype=np.int32)
    q = k = v = None
    if tensors:
        q, k, v = _draw_tensors(seed, branches, pool_pages, num_qo_heads, num_kv_heads, page_size, head_dim, dtype)
        pages = list(prefix_pages) + list(suf_indices)
        slots = [page_size] * n_prefix_pages + _used_slots(suf_indptr, suf_indices, suf_last, page_size)[1]
        _poison_unused(k, pages, slots)
        _poison_unused(v, pages, slots)
    formats = [
        Format(
            qo_indptr=np.array([0, branches], dtype=np.int32),
            kv_indptr=np.array([0, n_prefix_pages], dtype=np.int32),
            last_page_len=np.array([page_size], dtype=np.int32),
            kv_indices_offset=0,
        ),
        Format(
            qo_indptr=qo_indptr.copy(),
            kv_indptr=suf_indptr,
            last_page_len=suf_last,
            kv_indices_offset=n_prefix_pages,
        ),
    ]
    kv_indices_formats = np.concatenate([prefix_pages, suf_indices]).astype(np.int32)
    return Workload(
        name="shared_prefix_composable",
        dtype=dtype,
        num_qo_heads=num_qo_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        page_size=page_size,
        causal=False,
        cap=0.0,
        scale=1.0 / math.sqrt(head_dim),
        qo_indptr=qo_indptr,
        kv_indptr=np.asarray(single_indptr, dtype=np.int32),
        kv_indices=single_indices,
        last_page_len=suf_last.astype(np.int32),
        q=q,
        k_pool=k,
        v_pool=v,
        formats=formats,
        kv_indices_formats=kv_indices_formats,
    )


def quest_sparse_decode(seed=8, batch=1, seq=32768, page_size=16, num_heads=32, head_dim=128, tensors=True):
    """Long-context decode for Quest-style page budgets: the shape the explainer
    page quotes (sequence 32768, pages of 16 keys, 32 query and 32 KV heads, head
    dim 128), bf16, one query token per request."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return build("quest_sparse_decode", seed, [1] * batch, [seq] * batch, page_size, num_heads, num_heads, head_dim,
                 dtype="bf16", rng=rng, tensors=tensors)


def spec_decode_tree(seed=9, batch=32, lo=512, hi=8192, draft_lo=2, draft_hi=8, tensors=True):
    """Speculative decoding with token trees: batch decode shapes (32/8 heads,
    D=128, P=16, KV U[lo, hi]) with U[draft_lo, draft_hi] draft tokens per request
    that are the request's last keys; the tree masks are drawn by the caller."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kv = rng.integers(lo, hi, size=batch, endpoint=True)
    qo = rng.integers(draft_lo, draft_hi, size=batch, endpoint=True)
    return build("spec_decode_tree", seed, qo, kv, 16, 32, 8, 128, dtype="bf16", causal=True, rng=rng,
                 tensors=tensors)


def draft_trees(qo_lens, seed):
    """Token trees for speculative decoding, one boolean [n, n] matrix per request:
    draft token t (t > 0) hangs under a uniformly drawn earlier token or under the
    accepted prefix, and sees itself and its ancestors."""
    rng = np.random.Generator(np.random.PCG64(seed))
    trees = []
    for n in qo_lens:
        n = int(n)
        parent = [-1] + [int(rng.integers(-1, t)) for t in range(1, n)]
        m = np.zeros((n, n), dtype=bool)
        for t in range(n):
            u = t
            while u >= 0:
                m[t, u] = True
                u = parent[u]
        trees.append(m)
    return trees


NAMED = {
    "tiny_decode_f32": tiny_decode_f32,
    "batch_decode": batch_decode,
    "batch_decode_fp8": batch_decode_fp8,
    "batch_decode_window": batch_decode_window,
    "skewed_long_decode": skewed_long_decode,
    "ragged_causal_prefill": ragged_causal_prefill,
    "shared_prefix_composable": shared_prefix_composable,
    "ragged_causal_prefill_fp8": ragged_causal_prefill_fp8,
    "quest_sparse_decode": quest_sparse_decode,
    "spec_decode_tree": spec_decode_tree,
}


def named(name, **kw):
    return NAMED[name](**kw)
