"""ALiBi and tree-mask plans through a host-only handle (no GPU): the CPU float64
executor runs the decoded plan (positions and tree rows as the plan carries them)
and must reproduce the oracle; the plan call validates tree masks."""

import numpy as np
import pytest

import oracle
from serving_attention_bsr_amd import lib
from serving_attention_bsr_amd import workloads as W
from tests import plan_blob
from tests.variant_pins import random_tree


def host_handle(h_qo, h_kv, d, P, causal=False, cap=0.0, nwg=8, **kw):
    args = dict(num_qo_heads=h_qo, num_kv_heads=h_kv, head_dim=d, page_size=P, dtype="bf16", causal=causal,
                logits_soft_cap=cap, num_workgroups=nwg, device=-1, max_batch=64, max_total_qo=4096,
                max_total_kv=1 << 20)
    args.update(kw)
    return lib.BsrAttention(**args)


def f64(t):
    return t.double().numpy()


CASES = [
    # name, qo_lens, kv_lens, h_qo, h_kv, d, P, causal, cap, nwg, alibi, tree
    ("alibi_decode_split", [1, 1, 1], [300, 17, 1000], 8, 2, 64, 16, False, 0.0, 16, True, False),
    ("alibi_prefill_causal", [40, 7, 70], [100, 7, 200], 8, 2, 64, 1, True, 0.0, 8, True, False),
    ("alibi_cap_noncausal", [33, 1], [90, 450], 4, 1, 64, 2, False, 2.0, 5, True, False),
    ("tree_decode_rows", [2, 1, 2, 1], [50, 9, 300, 2], 8, 2, 64, 4, True, 0.0, 8, False, True),
    ("tree_wide_split", [16, 5, 64], [400, 5, 900], 8, 2, 64, 16, True, 0.0, 16, False, True),
    ("tree_noncausal_alibi_cap", [6, 3], [40, 700], 4, 2, 64, 3, False, 3.0, 8, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_variant_plan_executes_to_oracle(case):
    name, qo, kv, h_qo, h_kv, d, P, causal, cap, nwg, use_alibi, use_tree = case
    w = W.build(name, 17, qo, kv, P, h_qo, h_kv, d, causal=causal, cap=cap)
    rng = np.random.default_rng(4)
    slopes = rng.uniform(-0.5, 0.5, h_qo) if use_alibi else None
    trees = [random_tree(rng, n) for n in qo] if use_tree else None
    h = host_handle(h_qo, h_kv, d, P, causal, cap, nwg, alibi_slopes=slopes)
    if use_tree:
        h.plan_tree_mask(w.qo_indptr, w.kv_indptr, w.last_page_len, trees)
    else:
        h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    plan = plan_blob.decode(h.plan_bytes())
    q, k, v = f64(w.q), f64(w.k_pool), f64(w.v_pool)
    o, lse, written = plan_blob.execute(plan, q, k, v, w.kv_indices, w.group, P, w.scale, cap, alibi_slopes=slopes)
    ro, rl = oracle.bsr_attention(q, k, v, w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, P, h_qo, h_kv,
                                  w.scale, causal, cap, alibi_slopes=slopes, tree_masks=trees)
    assert np.all(written == 1)
    np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], rl[fin], rtol=1e-12, atol=1e-12)
    if use_alibi:
        stored = np.frombuffer(h.plan_bytes()[plan["header"]["off_alibi"]:][: 4 * h_qo].tobytes(), dtype="<f4")
        np.testing.assert_allclose(stored * w.scale, slopes, rtol=1e-6)


def test_tree_mask_rows_follow_the_packed_bits():
    qo, kv = [3, 1, 2], [10, 4, 2]
    w = W.build("tree_bits", 18, qo, kv, 4, 4, 2, 64, tensors=False)
    masks = [np.array([[1, 0, 0], [1, 1, 0], [1, 0, 1]], bool), np.array([[1]], bool), np.array([[1, 0], [0, 1]], bool)]
    h = host_handle(4, 2, 64, 4)
    h.plan_tree_mask(w.qo_indptr, w.kv_indptr, w.last_page_len, masks)
    plan = plan_blob.decode(h.plan_bytes())
    assert list(plan["tree"][:6]) == [0b001, 0b011, 0b101, 0b1, 0b01, 0b10]
    for it in plan["items"]:
        r = int(np.searchsorted(w.qo_indptr, int(it["qo_begin"]), side="right")) - 1
        assert int(it["tree_lo"]) == kv[r] - qo[r]


@pytest.mark.parametrize("qo, kv, code", [
    ([65], [100], lib.BSR_ERR_UNSUPPORTED),   # more than 64 tree tokens
    ([5], [3], lib.BSR_ERR_INVALID_ARG),      # more tree tokens than keys
])
def test_tree_mask_plan_rejects(qo, kv, code):
    w = W.build("tree_bad", 19, qo, kv, 4, 4, 2, 64, tensors=False)
    h = host_handle(4, 2, 64, 4)
    with pytest.raises(lib.BsrError) as e:
        h.plan_tree_mask(w.qo_indptr, w.kv_indptr, w.last_page_len, [np.ones((n, n), bool) for n in qo])
    assert e.value.code == code


def test_alibi_rejects_composed_formats_and_bad_slopes():
    h = host_handle(4, 2, 64, 4, alibi_slopes=[0.1, 0.2, 0.3, 0.4])
    fmt = dict(qo_indptr=np.array([0, 1], dtype=np.int32), kv_indptr=np.array([0, 1], dtype=np.int32),
               last_page_len=np.array([4], dtype=np.int32), kv_indices_offset=0)
    with pytest.raises(lib.BsrError) as e:
        h.plan_composable([fmt], 1)
    assert e.value.code == lib.BSR_ERR_UNSUPPORTED
    with pytest.raises(lib.BsrError) as e:
        host_handle(4, 2, 64, 4, alibi_slopes=[0.1, float("nan"), 0.3, 0.4])
    assert e.value.code == lib.BSR_ERR_INVALID_ARG
