"""Helpers for GPU tests: run a workload through the C ABI, compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from serving_attention_bsr_amd import lib

# Tolerances: O elementwise |o - ref| <= atol + rtol |ref|, LSE absolute.
TOL = {"bf16": (1e-2, 1e-2), "f32": (2e-5, 2e-5), "bf16_kv_fp8": (1e-2, 1e-2)}
LSE_TOL = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def handle_for(w, **kw):
    args = dict(
        num_qo_heads=w.num_qo_heads,
        num_kv_heads=w.num_kv_heads,
        head_dim=w.head_dim,
        page_size=w.page_size,
        dtype=w.dtype,
        causal=w.causal,
        logits_soft_cap=w.cap,
        sliding_window=w.window,
        max_batch=max(w.batch, 1) + (len(w.formats[1].qo_indptr) if w.formats else 0),
        max_total_qo=max(int(w.qo_indptr[-1]), 1),
        max_total_kv=max(int(w.kv_lens.sum()), 1),
        device=0,
    )
    args.update(kw)
    return lib.BsrAttention(**args)


def to_gpu(w):
    dev = torch.device("cuda:0")
    return (
        w.q.to(dev),
        w.k_pool.to(dev),
        w.v_pool.to(dev),
        torch.from_numpy(np.ascontiguousarray(w.kv_indices)).to(dev),
    )


def run_gpu(w, h=None, composable=False, **kw):
    """Plan and run workload w on cuda:0; returns (O float64 numpy, LSE numpy, info)."""
    h = h or handle_for(w, **kw)
    q, k, v, idx = to_gpu(w)
    if composable:
        info = h.plan_composable([f.as_dict() for f in w.formats], w.batch)
        idx = torch.from_numpy(np.ascontiguousarray(w.kv_indices_formats)).to(q.device)
    else:
        info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
    o, lse = h.run(q, k, v, idx)
    torch.cuda.synchronize()
    h.check()
    return o.double().cpu().numpy(), lse.double().cpu().numpy(), info


def oracle_of(w, composable=False, alibi_slopes=None, tree_masks=None):
    q = w.q.double().numpy()
    if w.k_pool.dtype == torch.float8_e4m3fn:
        # the oracle decodes the E4M3 codes itself
        k = oracle.decode_e4m3(w.k_pool.view(torch.uint8).numpy())
        v = oracle.decode_e4m3(w.v_pool.view(torch.uint8).numpy())
    else:
        k = w.k_pool.float().numpy()
        v = w.v_pool.float().numpy()
    if composable:
        return oracle.composable_attention(
            q, k, v, [f.as_dict() for f in w.formats], w.kv_indices_formats, w.page_size,
            w.num_qo_heads, w.num_kv_heads, w.scale, w.cap,
        )
    return oracle.bsr_attention(
        q, k, v, w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, w.page_size,
        w.num_qo_heads, w.num_kv_heads, w.scale, w.causal, w.cap, w.window,
        alibi_slopes=alibi_slopes, tree_masks=tree_masks,
    )


def compare(w, o, lse, ro, rl, label=""):
    atol, rtol = TOL[w.dtype]
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    err = np.abs(o - ro)
    bad = err > atol + rtol * np.abs(ro)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lse)), f"{label}: LSE finiteness differs"
    lerr = np.abs(lse[fin] - rl[fin]) if fin.any() else np.zeros(1)
    big = np.abs(ro) >= 1e-2
    stats = dict(
        max_abs_o=float(err.max()) if err.size else 0.0,
        max_rel_o=float((err[big] / np.abs(ro[big])).max()) if big.any() else 0.0,
        max_abs_lse=float(lerr.max()),
    )
    say(label, stats)
    assert not bad.any(), f"{label}: {int(bad.sum())} O elements outside tolerance {stats}"
    assert stats["max_abs_lse"] <= LSE_TOL, f"{label}: LSE {stats}"
    return stats
