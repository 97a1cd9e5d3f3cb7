"""GPU parity of bsr_attn_append_kv (writing new K/V rows into the paged cache)
against the CPU oracle, bit for bit (pure indexing).

Cases: decode appends (one row per request), whole-request prefill appends with
one key per page, a ragged mix with an empty request and a request with more new
rows than positions, D = 256 with an odd page size, a long prefill whose rows
cross requests inside one wavefront's range (more rows than wavefronts), and
page ids outside the pool
(those rows must not be written), and FP8 (E4M3) caches.  Pools start with random values everywhere, so
any write outside the expected slots shows up.
"""

import numpy as np
import pytest
import torch

import oracle
from serving_attention_bsr_amd import lib

CASES = [
    # name, kv lens after the write, new rows per request, H_kv, D, P, dtype, seed
    ("decode_p16", [int(x) for x in np.random.default_rng(1).integers(1, 300, 16)], [1] * 16, 8, 128, 16, "bf16", 1),
    ("prefill_p1", [5, 100, 33], [5, 100, 33], 4, 128, 1, "bf16", 2),
    ("ragged_f32_p3_overflow", [10, 4, 0, 7], [3, 6, 0, 7], 2, 64, 3, "f32", 3),
    ("d256_p5", [40, 41], [17, 1], 2, 256, 5, "bf16", 4),
    ("long_prefill_p16", [1000, 4000, 2500, 3100, 1, 2999, 3500, 2900], [1000, 4000, 2500, 3100, 1, 2999, 3500, 2900],
     8, 128, 16, "bf16", 5),
    # more new rows than the grid has wavefronts (65536): each wavefront walks two
    # tokens, across request boundaries
    ("many_tokens_h1", [30000, 25001, 19999], [30000, 25001, 19999], 1, 64, 16, "bf16", 6),
    # FP8 (E4M3) cache: one byte per element, 16-byte pieces of 16 elements
    ("fp8_decode_p16", [int(x) for x in np.random.default_rng(7).integers(1, 300, 16)], [1] * 16, 8, 128, 16, "fp8",
     7),
    ("fp8_prefill_p1_d64", [5, 100, 33], [5, 100, 33], 4, 64, 1, "fp8", 8),
    ("fp8_ragged_d256_p5_overflow", [10, 4, 0, 47], [3, 6, 0, 17], 2, 256, 5, "fp8", 9),
]


def _case(lens, new, h_kv, d, page_size, dtype, seed, spare=3):
    rng = np.random.default_rng(seed)
    n_pages = [(l + page_size - 1) // page_size for l in lens]
    num_pages = sum(n_pages) + spare
    order = rng.permutation(num_pages)
    kv_indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
    kv_indices = order[: sum(n_pages)].astype(np.int32)
    last = np.array([l - (n - 1) * page_size if n > 0 else page_size for l, n in zip(lens, n_pages)], dtype=np.int32)
    append_indptr = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.float8_e4m3fn}[dtype]
    g = torch.Generator().manual_seed(seed)
    k_pool = torch.randn((num_pages, h_kv, page_size, d), generator=g).to(tdt)
    v_pool = torch.randn((num_pages, h_kv, page_size, d), generator=g).to(tdt)
    k_new = torch.randn((int(append_indptr[-1]), h_kv, d), generator=g).to(tdt)
    v_new = torch.randn((int(append_indptr[-1]), h_kv, d), generator=g).to(tdt)
    return k_pool, v_pool, k_new, v_new, append_indptr, kv_indptr, kv_indices, last


def _bits(t):
    view = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.float8_e4m3fn: torch.uint8}[t.dtype]
    return t.view(view).numpy()


def _gpu_append(k_pool, v_pool, k_new, v_new, append_indptr, kv_indptr, kv_indices, last):
    dev = torch.device("cuda:0")
    kp, vp = k_pool.to(dev), v_pool.to(dev)
    idx = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
           for a in (append_indptr, kv_indptr, kv_indices, last)]
    lib.append_kv(k_new.to(dev), v_new.to(dev), *idx, kp, vp)
    torch.cuda.synchronize()
    return kp.cpu(), vp.cpu()


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_append_matches_oracle(case):
    name, lens, new, h_kv, d, page_size, dtype, seed = case
    print(f"case {name}", flush=True)
    k_pool, v_pool, k_new, v_new, append_indptr, kv_indptr, kv_indices, last = _case(lens, new, h_kv, d, page_size,
                                                                                    dtype, seed)
    ek, ev = oracle.append_paged_kv(_bits(k_pool), _bits(v_pool), _bits(k_new), _bits(v_new), append_indptr,
                                    kv_indptr, kv_indices, last, page_size)
    gk, gv = _gpu_append(k_pool, v_pool, k_new, v_new, append_indptr, kv_indptr, kv_indices, last)
    assert np.array_equal(_bits(gk), ek), name
    assert np.array_equal(_bits(gv), ev), name


@pytest.mark.gpu
def test_append_skips_pages_outside_the_pool():
    print("case pages_outside_pool", flush=True)
    lens, new, h_kv, d, page_size = [20, 9, 30], [4, 9, 2], 2, 128, 8
    k_pool, v_pool, k_new, v_new, append_indptr, kv_indptr, kv_indices, last = _case(lens, new, h_kv, d, page_size,
                                                                                    "bf16", 9, spare=0)
    num_pages = k_pool.shape[0]
    # request 1's pages point past the pool: the oracle writes them into extra pages
    # that the GPU does not have, so the GPU pool must equal the oracle's first pages
    bad = kv_indices.copy()
    bad[kv_indptr[1]:kv_indptr[2]] = num_pages + np.arange(kv_indptr[2] - kv_indptr[1])
    extra = int(kv_indptr[2] - kv_indptr[1])
    pad = lambda t: np.concatenate([_bits(t), np.zeros((extra,) + tuple(t.shape[1:]), dtype=_bits(t).dtype)])
    ek, ev = oracle.append_paged_kv(pad(k_pool), pad(v_pool), _bits(k_new), _bits(v_new), append_indptr, kv_indptr,
                                    bad, last, page_size)
    gk, gv = _gpu_append(k_pool, v_pool, k_new, v_new, append_indptr, kv_indptr, bad, last)
    assert np.array_equal(_bits(gk), ek[:num_pages])
    assert np.array_equal(_bits(gv), ev[:num_pages])


@pytest.mark.gpu
def test_append_graph_replays():
    """bsr_attn_append_kv captured in a HIP graph: every replay (with eager work and
    new rows in between) writes what the eager call writes."""
    print("case append_graph", flush=True)
    lens, new, h_kv, d, page_size = [300, 17, 64, 1000], [1, 17, 5, 40], 8, 128, 16
    k_pool, v_pool, k_new, v_new, append_indptr, kv_indptr, kv_indices, last = _case(lens, new, h_kv, d, page_size,
                                                                                    "bf16", 12)
    dev = torch.device("cuda:0")
    kp, vp = k_pool.to(dev), v_pool.to(dev)
    kn, vn = k_new.to(dev), v_new.to(dev)
    idx = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
           for a in (append_indptr, kv_indptr, kv_indices, last)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lib.append_kv(kn, vn, *idx, kp, vp)  # warm the launch path outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lib.append_kv(kn, vn, *idx, kp, vp)
    for rep in range(3):
        # fresh rows each time; restore the pools, replay, compare with the oracle
        kn.copy_(torch.randn(kn.shape, generator=torch.Generator().manual_seed(100 + rep)).to(kn.dtype))
        vn.copy_(-kn)
        kp.copy_(k_pool)
        vp.copy_(v_pool)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ek, ev = oracle.append_paged_kv(_bits(k_pool), _bits(v_pool), _bits(kn.cpu()), _bits(vn.cpu()),
                                        append_indptr, kv_indptr, kv_indices, last, page_size)
        assert np.array_equal(_bits(kp.cpu()), ek), f"replay {rep}"
        assert np.array_equal(_bits(vp.cpu()), ev), f"replay {rep}"
