"""Early release of partial states on the GPU (Core mechanism 6 of the FlashInfer
explainer page, paper Algorithm 1: merges wait on ready stamps).  Decode and mixed
grids run a queue's partial items first and stamp each one that is not the queue's
last right after it.  Each case's plan holds such items; the result must match the
oracle and repeat bit for bit (the merges still fold their sources in map order)."""

import numpy as np
import pytest
import torch

from serving_attention_bsr_amd import workloads as W
from tests import plan_blob
from tests.gpu_common import compare, handle_for, oracle_of, say, to_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # name, builder, num_workgroups, expected kernel kind
    ("skewed_small_32", lambda: W.named("skewed_long_decode", long_len=16384, n_short=7), 32, 1),
    ("decode_cap_16", lambda: W.build("decode_cap_16", 32, [1] * 6, [9000, 100, 200, 300, 5000, 64], 16, 32, 8, 128,
                                      dtype="bf16", cap=20.0), 16, 1),
    ("mixed_16", lambda: W.build("mixed_16", 31, [1, 1, 30, 1], [12000, 9000, 700, 300], 16, 16, 4, 128,
                                 dtype="bf16", causal=True), 16, 3),
    ("mixed_24", lambda: W.build("mixed_24", 31, [1, 1, 30, 1], [12000, 9000, 700, 300], 16, 16, 4, 128,
                                 dtype="bf16", causal=True), 24, 3),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_early_release_matches_oracle_and_repeats(case):
    name, build, nwg, kind = case
    say("case", name)
    w = build()
    h = handle_for(w, num_workgroups=nwg)
    q, k, v, idx = to_gpu(w)
    info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    say("plan", info)
    items = plan_blob.decode(h.plan_bytes())["items"]
    assert info["kernel"] == kind
    assert ((items["flags"] & plan_blob.ITEM_RELEASE) != 0).any(), "the plan must release some states early"
    o0, l0 = h.run(q, k, v, idx)
    o0, l0 = o0.clone(), l0.clone()
    for _ in range(3):
        o, l = h.run(q, k, v, idx)
        assert torch.equal(o.view(torch.int16), o0.view(torch.int16))
        assert torch.equal(l.view(torch.int32), l0.view(torch.int32))
    torch.cuda.synchronize()
    h.check()
    ro, rl = oracle_of(w)
    compare(w, o0.double().cpu().numpy(), l0.double().cpu().numpy(), ro, rl, name)
