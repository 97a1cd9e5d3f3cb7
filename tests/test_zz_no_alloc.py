"""bsr_attn_run_static (the entry point that allocates nothing: its workspace is
the library's static device array) against bsr_attn_run on the same plan, bit for
bit, on consecutive calls of decreasing size, through the C ABI (needs an
MI355X)."""

import numpy as np
import pytest
import torch

from serving_attention_bsr_amd import lib
from serving_attention_bsr_amd import workloads as W
from tests.gpu_common import compare, oracle_of, say, to_gpu

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).clone()


def _handle(w, **kw):
    args = dict(dtype=w.dtype, causal=w.causal, logits_soft_cap=w.cap, max_batch=16, max_total_qo=4096,
                max_total_kv=1 << 18, device=0, max_partial_rows=16384)
    args.update(kw)
    return lib.BsrAttention(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, **args)


def _both(h, w):
    q, k, v, idx = to_gpu(w)
    info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    o_ref, l_ref = h.run(q, k, v, idx)
    torch.cuda.synchronize()
    h.check()
    h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len, upload=False)
    o = torch.full_like(q, 3.0)
    lse = torch.full((q.shape[0], q.shape[1]), 3.0, dtype=torch.float32, device=q.device)
    h.run_static(q, k, v, idx, o, lse)
    torch.cuda.synchronize()
    h.check(static=True)
    assert torch.equal(_bits(o), _bits(o_ref)) and torch.equal(_bits(lse), _bits(l_ref)), w.name
    ro, rl = oracle_of(w)
    compare(w, o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, f"run_static {w.name}")
    return info


def test_run_static_matches_run_on_consecutive_calls():
    big = W.named("skewed_long_decode", long_len=16384, n_short=7)
    small = W.named("skewed_long_decode", long_len=3000, n_short=3)
    h = _handle(big)
    ws, _ = lib.bsr_attn_workspace_size(h.handle)
    say("workspace bytes", ws)
    assert ws <= 64 << 20
    i1 = _both(h, big)
    i2 = _both(h, small)
    say("plans", i1, i2)
    assert i1["num_merge_tasks"] > 0 and i2["num_items"] < i1["num_items"]


def test_run_static_mfma_then_smaller_prefill():
    mk = lambda seed, qo, kv: W.build(f"static_prefill_{seed}", seed, qo, kv, 1, 32, 8, 128, dtype="bf16",
                                      causal=True)
    h = _handle(mk(50, [64, 100], [6000, 3000]), num_workgroups=64)
    i1 = _both(h, mk(50, [64, 100], [6000, 3000]))
    i2 = _both(h, mk(51, [40], [900]))
    assert i1["kernel"] == lib.KERNEL_MFMA and i1["num_partial_items"] > 0


def test_run_static_rejects_a_workspace_beyond_the_scratch():
    w = W.named("tiny_decode_f32")
    h = lib.BsrAttention(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, dtype=w.dtype, device=0,
                         max_batch=4, max_total_qo=4, max_total_kv=1024, max_partial_rows=1 << 22)
    q, k, v, idx = to_gpu(w)
    h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len, upload=False)
    with pytest.raises(lib.BsrError) as e:
        h.run_static(q, k, v, idx)
    assert e.value.code == lib.BSR_ERR_CAPACITY
