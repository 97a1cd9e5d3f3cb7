"""GPU parity of the decode body over an FP8 (OCP E4M3) K/V cache with bf16 Q/O.

The oracle decodes the same E4M3 codes the GPU reads (oracle.decode_e4m3, pinned
against the format) and runs the plain attention definition; the tolerance is the
bf16 one.  Cases: head dims 64 / 128 / 256, split chunks with a soft-cap, 8-row
speculative decode, wide query rows on the MFMA tile body (head dims 64 and 128:
causal, one-key pages, soft-cap, splits, a mixed grid) or as 8-row decode tiles
(head dim 256), the batch decode workload and the ragged causal prefill with an
FP8 cache.
"""

import pytest

from serving_attention_bsr_amd import workloads as W
from tests.gpu_common import compare, oracle_of, run_gpu, say

pytestmark = pytest.mark.gpu

CASES = [
    # name, qo_lens, kv_lens, h_qo, h_kv, d, P, causal, cap, nwg
    ("kv8_d128_p16", [1] * 9, [1, 2, 31, 32, 33, 511, 512, 513, 3000], 32, 8, 128, 16, False, 0.0, 0),
    ("kv8_d64_split_cap", [1] * 4, [17, 64, 100, 2550], 8, 2, 64, 16, False, 5.0, 16),
    ("kv8_d256_p7_split", [1] * 3, [10, 300, 900], 16, 4, 256, 7, False, 0.0, 8),
    ("kv8_rows8_spec_causal", [2, 2, 1], [90, 333, 5], 8, 2, 128, 16, True, 0.0, 0),
    # wide rows at head dim 256 still run as 8-row decode tiles
    ("kv8_d256_wide_rows_decode_tiles", [20, 3], [40, 300], 8, 2, 256, 16, True, 0.0, 8),
    # FP8 on the 32-row MFMA tile body (head dims 64 and 128)
    ("kv8_mfma_d64_causal_split", [20, 3], [40, 300], 8, 2, 64, 16, True, 0.0, 8),
    ("kv8_mfma_d128_causal_p1", [300, 77, 1000], [700, 77, 1500], 32, 8, 128, 1, True, 0.0, 0),
    ("kv8_mfma_d128_p16_cap_split", [64, 100], [6000, 3000], 32, 8, 128, 16, True, 30.0, 64),
    ("kv8_mfma_d64_p3_noncausal", [129, 64], [65, 300], 4, 4, 64, 3, False, 0.0, 0),
    ("kv8_mfma_d128_g8_p1_cap", [60, 200], [60, 900], 16, 2, 128, 1, False, 20.0, 0),
    ("kv8_mixed_decode_prefill", [1, 50, 1, 3], [500, 120, 77, 3], 32, 8, 128, 4, True, 0.0, 16),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_kv_fp8_sweep(case):
    name, qo, kv, h_qo, h_kv, d, P, causal, cap, nwg = case
    say("case", name)
    w = W.build(name, 31, qo, kv, P, h_qo, h_kv, d, dtype=W.KV_FP8, causal=causal, cap=cap)
    o, lse, info = run_gpu(w, num_workgroups=nwg)
    say("plan", info)
    ro, rl = oracle_of(w)
    compare(w, o, lse, ro, rl, name)


def test_batch_decode_fp8():
    say("workload batch_decode_fp8")
    w = W.named("batch_decode_fp8")
    o, lse, info = run_gpu(w)
    say("plan", info)
    ro, rl = oracle_of(w)
    compare(w, o, lse, ro, rl, "batch_decode_fp8")


def test_kv_fp8_repeat_is_bitwise():
    """The same plan gives the same bits on repeated runs (FP8 K/V, split chunks)."""
    import torch

    from tests.gpu_common import handle_for, to_gpu

    say("case kv8_repeat")
    w = W.build("kv8_repeat", 41, [1] * 6, [5000, 17, 900, 1, 64, 2100], 16, 32, 8, 128, dtype=W.KV_FP8)
    h = handle_for(w, num_workgroups=64)
    q, k, v, idx = to_gpu(w)
    h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    first = None
    for rep in range(5):
        o, lse = h.run(q, k, v, idx)
        torch.cuda.synchronize()
        h.check()
        if first is None:
            first = (o.clone(), lse.clone())
        else:
            assert torch.equal(o.view(torch.int16), first[0].view(torch.int16)), rep
            assert torch.equal(lse.view(torch.int32), first[1].view(torch.int32)), rep


def test_ragged_causal_prefill_fp8():
    say("workload ragged_causal_prefill_fp8")
    w = W.named("ragged_causal_prefill_fp8")
    o, lse, info = run_gpu(w)
    say("plan", info)
    assert info["kernel"] == 2
    ro, rl = oracle_of(w)
    compare(w, o, lse, ro, rl, "ragged_causal_prefill_fp8")
