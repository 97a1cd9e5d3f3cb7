"""Decoder of the plan bytes a host-only handle stages, and a CPU float64 executor.

The layout decoded here is the one documented in the library's layout header:
an 88-byte header of int32 counts, offsets, the kernel instance, the wait bound and the
first claimed item, then status words, claim counters, per-workgroup epochs, ready
flags, per-workgroup item queues (CSR), 64-byte work items (the queues' items, then
the pool that workgroups claim at run time), per-workgroup
merge queues (CSR), 16-byte merge tasks and 8-byte merge sources.

The executor runs the plan's work items and merge map with the oracle's
attention and ⊕ in float64; if the plan covers every (query, key) pair exactly
once and merges in a valid order, it reproduces the oracle's whole-request result.
"""

from __future__ import annotations

import numpy as np

import oracle

HEADER_FIELDS = [
    "magic", "kernel", "num_wg", "num_items", "num_merge", "num_srcs", "num_flags",
    "off_status", "off_epochs", "off_flags", "off_item_ptr", "off_items", "off_merge_ptr",
    "off_merge", "off_srcs", "blob_bytes", "instance", "spin_limit", "off_alibi", "off_tree", "pool_begin",
    "off_claim",
]
HEADER_BYTES = 4 * len(HEADER_FIELDS)
ITEM = np.dtype([
    ("flags", "<i4"), ("qo_begin", "<i4"), ("qo_count", "<i4"), ("kv_head", "<i4"),
    ("page_begin", "<i4"), ("kv_begin", "<i4"), ("kv_end", "<i4"), ("causal_limit", "<i4"),
    ("partial_row", "<i4"), ("flag_id", "<i4"), ("window_lo", "<i4"), ("q_pos", "<i4"), ("tree_lo", "<i4"),
    ("pad0", "<i4"), ("pad1", "<i4"), ("pad2", "<i4"),
])
NO_TREE = 0x3FFFFFFF
TASK = np.dtype([("qo_row", "<i4"), ("kv_head", "<i4"), ("src_begin", "<i4"), ("src_count", "<i4")])
SRC = np.dtype([("partial_row", "<i4"), ("flag_id", "<i4")])
ITEM_MFMA = 1
ITEM_PARTIAL = 2
ITEM_RELEASE = 4
MAGIC = 0x41525342


def decode(blob: np.ndarray) -> dict:
    blob = np.asarray(blob, dtype=np.uint8)
    hdr = dict(zip(HEADER_FIELDS, np.frombuffer(blob[:HEADER_BYTES].tobytes(), dtype="<i4").tolist()))
    assert hdr["magic"] == MAGIC
    nwg = hdr["num_wg"]

    def arr(off, dtype, n):
        return np.frombuffer(blob[off : off + np.dtype(dtype).itemsize * n].tobytes(), dtype=dtype)

    assert 0 <= hdr["pool_begin"] <= hdr["num_items"]
    tree = None
    if hdr["off_tree"]:
        end = hdr["off_tree"] + 8 * ((hdr["blob_bytes"] - hdr["off_tree"]) // 8)
        tree = np.frombuffer(blob[hdr["off_tree"] : end].tobytes(), dtype="<u8")
    return dict(
        tree=tree,
        header=hdr,
        epochs=arr(hdr["off_epochs"], "<i4", nwg),
        flags=arr(hdr["off_flags"], "<i4", hdr["num_flags"]),
        item_ptr=arr(hdr["off_item_ptr"], "<i4", nwg + 1),
        claims=arr(hdr["off_claim"], "<i4", 2),
        items=arr(hdr["off_items"], ITEM, hdr["num_items"]),
        merge_ptr=arr(hdr["off_merge_ptr"], "<i4", nwg + 1),
        merge=arr(hdr["off_merge"], TASK, hdr["num_merge"]),
        srcs=arr(hdr["off_srcs"], SRC, hdr["num_srcs"]),
    )


def execute(plan, q, k_pool, v_pool, kv_indices, group, page_size, scale, cap, alibi_slopes=None):
    """Run the decoded plan on the CPU in float64; returns O, LSE (natural log).

    Positions (ALiBi) and tree-mask rows come from the plan; the slopes are the
    caller's (the plan holds them divided by the scale, in float32)."""
    total, h_qo, d = q.shape
    out = np.zeros((total, h_qo, v_pool.shape[3]))
    lse = np.full((total, h_qo), -np.inf)
    partial = {}
    written = np.zeros((total, h_qo), dtype=np.int64)
    nwg = plan["header"]["num_wg"]
    # every item once: the per-workgroup queues, then the claimed pool (which
    # workgroup runs an item does not change its result)
    for it in plan["items"]:
        kb, ke = int(it["kv_begin"]), int(it["kv_end"])
        tau = np.arange(kb, ke)
        pages = kv_indices[int(it["page_begin"]) + tau // page_size]
        k = np.asarray(k_pool[pages, int(it["kv_head"]), tau % page_size, :], dtype=np.float64)
        v = np.asarray(v_pool[pages, int(it["kv_head"]), tau % page_size, :], dtype=np.float64)
        for t in range(int(it["qo_count"])):
            token = int(it["qo_begin"]) + t
            limit = int(it["causal_limit"]) + t
            vis = (tau <= limit) & (tau >= int(it["window_lo"]) + t)
            tlo = int(it["tree_lo"])
            if tlo != NO_TREE:
                row = np.uint64(plan["tree"][token])
                bit = np.clip(tau - tlo, 0, 63).astype(np.uint64)
                vis &= (tau < tlo) | (((row >> bit) & np.uint64(1)) == 1)
            for j in range(group):
                head = int(it["kv_head"]) * group + j
                bias = None
                if alibi_slopes is not None:
                    bias = (float(alibi_slopes[head]) * (tau[vis] - (int(it["q_pos"]) + t)))[None, :]
                o1, l1 = oracle.attention_dense(
                    np.asarray(q[token : token + 1, head, :], dtype=np.float64), k[vis], v[vis], scale, cap,
                    bias=bias,
                )
                if it["flags"] & ITEM_PARTIAL:
                    row = int(it["partial_row"]) + t * group + j
                    assert row not in partial, "partial row written twice"
                    partial[row] = (o1[0], l1[0], int(it["flag_id"]))
                else:
                    out[token, head] = o1[0]
                    lse[token, head] = l1[0]
                    written[token, head] += 1
    for w in range(nwg):
        for m in plan["merge"][plan["merge_ptr"][w] : plan["merge_ptr"][w + 1]]:
            srcs = plan["srcs"][int(m["src_begin"]) : int(m["src_begin"]) + int(m["src_count"])]
            for j in range(group):
                head = int(m["kv_head"]) * group + j
                states = []
                for s in srcs:
                    o1, l1, fid = partial[int(s["partial_row"]) + j]
                    assert fid == int(s["flag_id"]), "merge source waits on the wrong flag"
                    states.append((o1[None], np.array([l1])))
                if states:
                    o1, l1 = oracle.merge_states(states)
                    out[int(m["qo_row"]), head] = o1[0]
                    lse[int(m["qo_row"]), head] = l1[0]
                written[int(m["qo_row"]), head] += 1
    return out, lse, written
