"""Query tile height (Core mechanism 4 of the FlashInfer explainer page, paper
section 3.2.2): the planner takes the smallest tile of the kernel's menu that is at
least the mean folded length of the rows that need tiles.  The tile kernel at head
dim 128 with bf16 K/V offers 64 and 128 folded rows; every other kernel one height
(128 up to head dim 128, 64 at 256).  The 64-row tile is its own kernel instance,
so it shows in the plan's instance key (folded-rows field 1)."""

import numpy as np
import pytest

from serving_attention_bsr_amd import lib
from tests import plan_blob


def handle(h_qo=32, h_kv=8, d=128, dtype="bf16", **kw):
    args = dict(num_qo_heads=h_qo, num_kv_heads=h_kv, head_dim=d, page_size=16, dtype=dtype, num_workgroups=32,
                device=-1, max_batch=64, max_total_qo=8192, max_total_kv=1 << 20)
    args.update(kw)
    return lib.BsrAttention(**args)


def plan(h, qo_lens, kv_lens):
    qo = np.concatenate([[0], np.cumsum(qo_lens)])
    pages = [(k + 15) // 16 for k in kv_lens]
    kv = np.concatenate([[0], np.cumsum(pages)])
    last = [k - 16 * (p - 1) for k, p in zip(kv_lens, pages)]
    info = h.plan(qo, kv, last)
    return info, plan_blob.decode(h.plan_bytes())


def rows_field(instance):
    return (instance >> 4) & 15


@pytest.mark.parametrize(
    "qo_lens, tile",
    [
        ([16] * 8, 64),            # 64 folded rows each: exactly the short tile
        ([3, 5, 8, 16, 12], 64),   # draft-sized rows: mean 35.2 folded rows
        ([16, 17], 128),           # mean 66 folded rows
        ([300, 4, 4], 128),        # one long row pulls the mean above 64
        ([2048], 128),             # prefill
    ],
)
def test_tile_is_the_smallest_at_least_the_mean(qo_lens, tile):
    h = handle()
    info, p = plan(h, qo_lens, [4000] * len(qo_lens))
    assert info["kernel"] == 2
    assert info["q_tile"] == tile
    assert rows_field(info["instance"]) == (1 if tile == 64 else 0)
    assert p["header"]["instance"] == info["instance"]
    # every item covers at most one tile of folded rows of one row
    its = p["items"]
    assert (its["qo_count"] * 4 <= tile).all()


def test_other_kernels_keep_their_single_tile():
    short = [16] * 8
    # FP8 K/V: the 32-row body only
    info, _ = plan(handle(dtype="bf16_kv_fp8"), short, [4000] * 8)
    assert (info["kernel"], info["q_tile"], rows_field(info["instance"])) == (2, 128, 0)
    # head dim 256: 64-row tiles of the 16-row body, the kernel's one height
    info, _ = plan(handle(d=256), short, [4000] * 8)
    assert (info["kernel"], info["q_tile"], rows_field(info["instance"])) == (2, 64, 0)
    # the mixed grid (decode-sized rows stream a quarter of the KV tokens) keeps 128
    info, _ = plan(handle(), [1, 1, 16], [4000, 4000, 4000])
    assert (info["kernel"], info["q_tile"]) == (3, 128)


def test_short_tile_plans_cover_every_query_row_once():
    """Items of a 64-row-tile plan tile each row's tokens without gaps or overlap
    (per KV head, summed over the KV chunks' first items)."""
    h = handle()
    qo_lens = [3, 5, 8, 16, 12, 40]
    info, p = plan(h, qo_lens, [1000, 3000, 64, 9000, 17, 5000])
    assert info["q_tile"] == 64
    its = p["items"]
    qo = np.concatenate([[0], np.cumsum(qo_lens)])
    for head in range(8):
        cov = np.zeros(qo[-1], dtype=np.int64)
        m = (its["kv_head"] == head) & (its["kv_begin"] == 0)
        for it in its[m]:
            cov[it["qo_begin"]:it["qo_begin"] + it["qo_count"]] += 1
        assert (cov == 1).all()
