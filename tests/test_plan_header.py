"""The plan header names the kernel instance a plan is made for, and the default
partial-state capacity covers composed formats over several KV heads.

The persistent kernel compares the header's instance with its own template
arguments (kind, decode rows, head dim, switches) and refuses a plan made for
another instance, so a run captured for one plan never silently runs a later plan
that needs another instance.  The key is laid out as documented next to
instance_key() in the library's layout header.
"""

import numpy as np
import pytest

from serving_attention_bsr_amd import lib
from serving_attention_bsr_amd import workloads as W
from tests import plan_blob


def expected_key(kind, rows, d, bf16=True, cap=False, page1=False, kv8=False):
    return kind | (rows << 4) | ((d // 64) << 8) | (bf16 << 12) | (cap << 13) | (page1 << 14) | (kv8 << 15)


def handle(h_qo=32, h_kv=8, d=128, P=16, **kw):
    args = dict(num_qo_heads=h_qo, num_kv_heads=h_kv, head_dim=d, page_size=P, dtype="bf16", num_workgroups=16,
                device=-1, max_batch=64, max_total_qo=4096, max_total_kv=1 << 20)
    args.update(kw)
    return lib.BsrAttention(**args)


@pytest.mark.parametrize(
    "qo, kv, last, P, cap, kind, rows",
    [
        ([0, 1, 2], [0, 3, 5], [16, 4], 16, False, 1, 4),       # decode, g = 4: 4 folded rows
        ([0, 2, 3], [0, 3, 5], [16, 4], 16, True, 1, 8),        # a 2-token row needs the 8-row body
        ([0, 300], [0, 20], [16], 16, False, 2, 0),              # MFMA tiles only
        ([0, 300, 301], [0, 20, 95], [16, 16], 16, True, 3, 4),  # both bodies (27 % decode-row tokens)
        ([0, 64], [0, 90], [1], 1, False, 2, 0),                 # one key per page: its own instance
    ],
)
def test_header_carries_the_instance(qo, kv, last, P, cap, kind, rows):
    h = handle(P=P, logits_soft_cap=30.0 if cap else 0.0)
    info = h.plan(qo, kv, last)
    hdr = plan_blob.decode(h.plan_bytes())["header"]
    want = expected_key(kind, rows, 128, cap=cap, page1=(kind == 2 and P == 1))
    assert info["kernel"] == kind
    assert hdr["instance"] == info["instance"] == want
    assert hdr["spin_limit"] == 1 << 21


def test_instance_changes_with_decode_rows():
    """The speculative-decoding case: the same batch with one request at two tokens
    needs the 8-row decode body, so a run captured for the 1-token plan must not
    replay it."""
    h = handle()
    one = h.plan([0, 1, 2], [0, 3, 5], [16, 4])["instance"]
    two = h.plan([0, 1, 3], [0, 3, 5], [16, 4])["instance"]
    assert one != two


@pytest.mark.parametrize("branches", [64, 512, 2048])
def test_composable_partials_fit_the_default_capacity(branches):
    """Each composed token needs one partial state per format for every query head;
    the default capacity counts them (h_kv > 1, more tokens than the tile term)."""
    w = W.shared_prefix_composable(branches=branches, prefix_len=256, suf_lo=1, suf_hi=40, head_dim=128,
                                   tensors=False)
    fm = [f.as_dict() for f in w.formats]
    mb = w.batch + sum(len(f.qo_indptr) - 1 for f in w.formats)
    h = handle(num_workgroups=8, max_batch=mb, max_total_qo=branches, max_total_kv=int(w.kv_lens.sum()))
    info = h.plan_composable(fm, w.batch)
    assert info["num_partial_rows"] >= 2 * branches * 32 - 8 * 128


def test_host_plan_reports_info_without_upload():
    h = handle()
    info = h.plan([0, 1], [0, 2], [5])
    assert info["blob_bytes"] > 0
    with pytest.raises(lib.BsrError) as e:
        lib.bsr_attn_run(h.handle, None, None, None, None, None, None, None, None)
    assert e.value.code == lib.BSR_ERR_INVALID_ARG
