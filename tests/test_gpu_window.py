"""GPU parity of the sliding-window mask against the oracle.

The window is one of the mask variants of the FlashInfer explainer page
(Background, and paper section 3.2.3's LogitsMask functor); a query token sees
the W keys ending at its bottom-right aligned position.  Cases cover every body
that masks: the VALU decode body (bf16, fp32, FP8 K/V, soft-cap, chunks split by
a small grid), the 32-row MFMA body (one-key and 16-key pages), the 16-row D=256
MFMA body, a window of one key, non-causal windows and a window longer than the
KV.  The planner starts each tile at its window, so these runs also check that
the shortened chunks and their merges line up with the oracle.
"""

import pytest

from serving_attention_bsr_amd import workloads as W
from tests.gpu_common import compare, oracle_of, run_gpu, say

CASES = [
    # name, qo_lens, kv_lens, h_qo, h_kv, d, P, dtype, causal, cap, nwg, window
    ("win_decode_bf16_split", [1] * 6, [4000, 700, 64, 1, 300, 129], 32, 8, 128, 16, "bf16", False, 0.0, 16, 300),
    ("win_spec_f32", [2, 3, 1], [90, 333, 500], 8, 2, 64, 5, "f32", True, 0.0, 0, 37),
    ("win_decode_cap_d256", [1, 1, 1], [1000, 70, 2000], 16, 4, 256, 16, "bf16", False, 20.0, 0, 129),
    ("win_fp8_decode", [1] * 4, [3000, 100, 700, 1], 32, 8, 128, 16, "bf16_kv_fp8", True, 0.0, 0, 256),
    ("win_mfma_d128_causal_p1", [300, 33, 128], [700, 33, 1000], 32, 8, 128, 1, "bf16", True, 0.0, 8, 100),
    ("win_mfma_d128_p16", [200, 64], [2000, 64], 32, 8, 128, 16, "bf16", True, 0.0, 0, 513),
    ("win_mfma_d64_noncausal", [129, 64], [65, 300], 4, 4, 64, 16, "bf16", False, 0.0, 0, 40),
    ("win_mfma_d256_causal_split", [90, 17], [600, 17], 16, 4, 256, 1, "bf16", True, 0.0, 8, 77),
    ("win_one_mfma", [70, 5], [70, 80], 8, 2, 128, 3, "bf16", True, 0.0, 0, 1),
    ("win_longer_than_kv", [40, 1], [100, 64], 8, 2, 128, 16, "bf16", True, 0.0, 0, 5000),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_window_matches_oracle(case):
    name, qo, kv, h_qo, h_kv, d, P, dtype, causal, cap, nwg, window = case
    say("case", name)
    w = W.build(name, 31, qo, kv, P, h_qo, h_kv, d, dtype=dtype, causal=causal, cap=cap, window=window)
    o, lse, info = run_gpu(w, num_workgroups=nwg)
    say("plan", info)
    ro, rl = oracle_of(w)
    compare(w, o, lse, ro, rl, name)
