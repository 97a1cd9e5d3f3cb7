"""Benchmark of the BSR attention hot path on one MI355X.

A step is one run() of the persistent kernel over one batch of synthetic input
(plan done beforehand; its host time is reported separately, since one plan
serves every layer of a generation step).  Each timed step is preceded, outside
the timed window, by a read of a 1 GiB buffer that evicts L2 and the 256 MB
Infinity Cache (a read leaves no dirty lines whose write-back would land in the
timed kernel), and is timed with HIP events on the stream the kernel runs on.

The headline line is the batch decode workload (64 requests, KV 512..8192,
Llama-3-8B attention shape): achieved HBM bandwidth = algorithmic bytes / median
step time.  The other workloads are reported in "workloads" (decode: TB/s;
prefill: TFLOP/s).  The CPU oracle is timed on the same host as a baseline.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attn HBM TB/s (% peak) + ragged prefill TFLOPS (% MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 flop/clk (dense)
HEADLINE = "batch_decode"
ALL = ["tiny_decode_f32", "batch_decode", "skewed_long_decode", "ragged_causal_prefill", "shared_prefix_composable",
       "batch_decode_fp8", "ragged_causal_prefill_fp8", "batch_decode_window", "spec_decode_tree", "append_kv_prefill",
       "quest_sparse_decode"]
# workloads bound by the matrix cores (the rest by HBM)
MFMA_BOUND = ("ragged_causal_prefill", "ragged_causal_prefill_fp8")
# Quest-style page-budget decode: the step is the page choice plus attention
QUEST = {"quest_sparse_decode": 64}  # page budget
# writing the new K/V rows of a workload into its paged cache (not an attention run)
APPEND = {"append_kv_prefill": "ragged_causal_prefill"}


STATIC_QUEUES = False  # set by --static-queues


def kernel_source_hash():
    """sha256 over the library's kernel and host sources, in path order."""
    h = hashlib.sha256()
    base = os.path.join(ROOT, "serving_attention_bsr_amd", "csrc")
    for path in sorted(glob.glob(os.path.join(base, "**", "*"), recursive=True)):
        if path.endswith((".h", ".hpp", ".hip", ".cpp")):
            h.update(os.path.relpath(path, base).encode())
            with open(path, "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per launch from the committed counter record of this workload, or
    None when the record is missing or was taken from other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes")


def recorded_mfma_busy(workload):
    """Fraction of SIMD cycles the matrix cores were busy, from the committed counter
    record of this workload (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE), or None
    when the record is missing or was taken from other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{workload}_mfma_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("mfma_busy")


def roofline(work, ms, traffic, mfma, mfma_busy=None):
    """Roofline entry of one workload: decode bodies are bound by HBM bytes, MFMA
    tile bodies by bf16 matrix throughput (with the counters' MFMA-busy fraction)."""
    if mfma:
        achieved = work["flops"] / (ms * 1e-3) / 1e12
        return dict(bound="mfma", achieved=round(achieved, 1), peak=BF16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / BF16_MFMA_PEAK_TFLOPS, 4), traffic=traffic, mfma_busy=mfma_busy)
    achieved = work["bytes"] / (ms * 1e-3) / 1e9
    return dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic)


def algorithmic_work(w, composable=False):
    """Bytes the method must move and flops it must do (masked pairs excluded)."""
    elt = 2 if w.dtype == "bf16" else 4            # Q and O
    kv_elt = 1 if w.dtype == "bf16_kv_fp8" else 2 if w.dtype == "bf16" else 4
    if w.dtype == "bf16_kv_fp8":
        elt = 2
    h_qo, h_kv, d = w.num_qo_heads, w.num_kv_heads, w.head_dim
    total_qo = int(w.qo_indptr[-1])
    qol = w.qo_lens.astype(np.int64)
    if composable:
        keys = 0
        pages = 0
        for f in w.formats:
            n = np.diff(f.kv_indptr.astype(np.int64))
            lens = np.where(n > 0, (n - 1) * w.page_size + f.last_page_len.astype(np.int64), 0)
            keys += int(lens.sum())
            pages += int(n.sum())
        pair_count = int(np.sum(w.kv_lens * qol))  # every branch attends prefix + suffix
    elif w.window > 0:
        # a sliding window: the keys of a request are those its first token's window
        # reaches and beyond, its pairs the keys each token sees
        keys = pages = pair_count = 0
        for lq, lk in zip(qol, w.kv_lens.astype(np.int64)):
            pos = lk - lq + np.arange(lq)
            lo = np.maximum(pos - w.window + 1, 0)
            hi = pos + 1 if w.causal else np.full(lq, lk)
            if lq:
                keys += int(lk - lo[0])
                pages += int((lk + w.page_size - 1) // w.page_size - lo[0] // w.page_size)
                pair_count += int(np.sum(hi - lo))
    else:
        keys = int(w.kv_lens.sum())
        pages = int(np.diff(w.kv_indptr.astype(np.int64)).sum())
        if w.causal:
            prefix = w.kv_lens - qol
            pair_count = int(np.sum(qol * prefix + qol * (qol + 1) // 2))
        else:
            pair_count = int(np.sum(w.kv_lens * qol))
    kv_bytes = 2 * keys * h_kv * d * kv_elt
    qo_bytes = 2 * total_qo * h_qo * d * elt + total_qo * h_qo * 4
    idx_bytes = 4 * pages
    flops = 4 * d * h_qo * pair_count
    return dict(bytes=kv_bytes + qo_bytes + idx_bytes, kv_bytes=kv_bytes, flops=flops)


def flush_caches(flush, mode):
    """Evict L2 and the Infinity Cache: read (default) leaves only clean lines behind,
    so the timed kernel pays no write-back of the flush's own data."""
    if flush is None or mode == "none":
        return
    if mode == "write":
        flush.add_(1)
    else:
        flush.view(-1, 1 << 16).amax(dim=1)


def timed_steps(fn, steps, warmup, stream, flush, mode="read"):
    """Per-step HIP-event times (ms) of fn(), each preceded by a cache flush."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        flush_caches(flush, mode)
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return np.array([s.elapsed_time(e) for s, e in zip(starts, ends)]), wall


def bench_workload(name, steps, warmup, flush, graph=True, nwg=0, mode="read"):
    import torch

    from serving_attention_bsr_amd import lib
    from serving_attention_bsr_amd import workloads as W

    print(f"[bench] {name}: building inputs", file=sys.stderr, flush=True)
    w = W.named(name)
    composable = w.formats is not None
    dev = torch.device("cuda:0")
    q, k, v = w.q.to(dev), w.k_pool.to(dev), w.v_pool.to(dev)
    idx_host = w.kv_indices_formats if composable else w.kv_indices
    idx = torch.from_numpy(np.ascontiguousarray(idx_host)).to(dev)
    max_batch = w.batch + (sum(len(f.qo_indptr) - 1 for f in w.formats) if composable else 0)
    h = lib.BsrAttention(
        w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, dtype=w.dtype, causal=w.causal,
        logits_soft_cap=w.cap, max_batch=max_batch, max_total_qo=int(w.qo_indptr[-1]),
        max_total_kv=int(w.kv_lens.sum()), device=0, num_workgroups=nwg, sliding_window=w.window,
        static_queues=STATIC_QUEUES,
    )
    work = algorithmic_work(w, composable)
    out = dict(workload=name, dtype=w.dtype, bytes=work["bytes"], flops=work["flops"])
    trees = W.draft_trees(w.qo_lens, 10) if name == "spec_decode_tree" else None
    try:
        torch.cuda.synchronize()
        plan_times = []
        for _ in range(20):
            t0 = time.perf_counter()
            if composable:
                info = h.plan_composable([f.as_dict() for f in w.formats], w.batch)
            elif trees is not None:
                info = h.plan_tree_mask(w.qo_indptr, w.kv_indptr, w.last_page_len, trees)
            else:
                info = h.plan(w.qo_indptr, w.kv_indptr, w.last_page_len)
            plan_times.append(time.perf_counter() - t0)
        torch.cuda.synchronize()
        out["plan_us"] = float(np.median(plan_times) * 1e6)
        out["plan_us_first"] = float(plan_times[0] * 1e6)
    except lib.BsrError as exc:
        out["error"] = str(exc)
        return out, None
    out["plan"] = info
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        h.run(q, k, v, idx, o, lse)

    times, wall = timed_steps(step, steps, warmup, stream, flush, mode)
    h.check()
    med = float(np.median(times))
    out["ms_median"] = med
    out["ms_min"] = float(times.min())
    out["ms_mean"] = float(times.mean())
    out["wall_s"] = wall
    gbs = work["bytes"] / (med * 1e-3) / 1e9
    tfl = work["flops"] / (med * 1e-3) / 1e12
    out["hbm_GBps"] = gbs
    out["hbm_frac"] = gbs / HBM_PEAK_GBS
    out["tflops"] = tfl
    out["mfma_frac"] = tfl / BF16_MFMA_PEAK_TFLOPS
    # prefill is bound by the matrix cores; decode and the shared-prefix batch
    # (whose prefix is read once for all branches) by HBM
    out["roofline"] = roofline(work, med, recorded_traffic(name), mfma=name in MFMA_BOUND,
                               mfma_busy=recorded_mfma_busy(name))
    if graph:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(stream)
            with torch.cuda.stream(s):
                step()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step()
            gt, _ = timed_steps(g.replay, steps, warmup, stream, flush, mode)
            out["graph_ms_median"] = float(np.median(gt))
            # a graph launch has a fixed cost of its own (its start and end in the
            # runtime); ten runs in one graph against ten eager runs, per run (one
            # cache flush before each group of ten)
            g10 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g10, stream=s):
                for _ in range(10):
                    step()
            gt10, _ = timed_steps(g10.replay, max(steps // 4, 3), 2, stream, flush, mode)
            et10, _ = timed_steps(lambda: [step() for _ in range(10)], max(steps // 4, 3), 2, stream, flush, mode)
            out["graph10_ms_per_run"] = float(np.median(gt10)) / 10
            out["eager10_ms_per_run"] = float(np.median(et10)) / 10
        except Exception as exc:  # report, do not hide
            out["graph_error"] = repr(exc)
    return out, (w, h)


def bench_append(name, steps, warmup, flush, mode="read"):
    """bsr_attn_append_kv over a workload's new tokens: their K/V rows ([sum l_qo,
    H_kv, D]) go to the last positions of each request in its page table.  Bound by
    HBM: every row is read once and written once."""
    import torch

    from serving_attention_bsr_amd import lib
    from serving_attention_bsr_amd import workloads as W

    src = APPEND[name]
    print(f"[bench] {name}: building inputs ({src} page table)", file=sys.stderr, flush=True)
    w = W.named(src)
    dev = torch.device("cuda:0")
    k_pool, v_pool = w.k_pool.to(dev), w.v_pool.to(dev)
    total_new = int(w.qo_indptr[-1])
    g = torch.Generator(device=dev).manual_seed(7)
    shape = (total_new, w.num_kv_heads, w.head_dim)
    k_new = torch.randn(shape, generator=g, device=dev).to(k_pool.dtype)
    v_new = torch.randn(shape, generator=g, device=dev).to(k_pool.dtype)
    idx = [torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
           for a in (w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len)]
    elt = k_pool.element_size()
    row_bytes = total_new * w.num_kv_heads * w.head_dim * elt
    work_bytes = 2 * 2 * row_bytes + 4 * (len(w.qo_indptr) + 2 * len(w.kv_indptr) + total_new)
    stream = torch.cuda.current_stream()

    def step():
        lib.append_kv(k_new, v_new, *idx, k_pool, v_pool)

    times, wall = timed_steps(step, steps, warmup, stream, flush, mode)
    med = float(np.median(times))
    gbs = work_bytes / (med * 1e-3) / 1e9
    return dict(workload=name, dtype=w.dtype, rows=total_new * w.num_kv_heads, bytes=work_bytes,
                ms_median=med, ms_min=float(times.min()), wall_s=wall, hbm_GBps=gbs, hbm_frac=gbs / HBM_PEAK_GBS,
                roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None)), None


def bench_quest(name, steps, warmup, flush, mode="read", graph=True):
    """Quest-style sparse decode at the page's shape: one step is the page choice
    (scores from the per-page key summaries, top pages per request and KV head) and
    attention over the kept pages (run() of the per-head plan, made once from the
    lengths).  The summaries are built before timing: they change only when a page
    fills.  Algorithmic bytes: the summaries (2 D elements per page and KV head),
    the kept K/V, Q, O and LSE."""
    import torch

    from serving_attention_bsr_amd import lib
    from serving_attention_bsr_amd import workloads as W

    budget = QUEST[name]
    print(f"[bench] {name}: building inputs", file=sys.stderr, flush=True)
    w = W.named(name)
    dev = torch.device("cuda:0")
    q, k, v = w.q.to(dev), w.k_pool.to(dev), w.v_pool.to(dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    kvp, kvi, last = i32(w.kv_indptr), i32(w.kv_indices), i32(w.last_page_len)
    kmin, kmax = lib.page_summary(k, kvp, kvi, last)
    out_ptr_h = lib.quest_out_indptr(w.kv_indptr, w.num_kv_heads, budget)
    out_ptr = i32(out_ptr_h)
    out_idx = torch.empty(int(out_ptr_h[-1]), dtype=torch.int32, device=dev)
    scores = torch.empty(w.num_kv_heads * len(w.kv_indices), dtype=torch.float32, device=dev)
    n_max = int(np.diff(w.kv_indptr).max())
    h = lib.BsrAttention(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size, dtype=w.dtype,
                         max_batch=w.batch, max_total_qo=w.batch, max_total_kv=int(w.kv_lens.max()), device=0)
    plan_times = []
    for _ in range(20):
        t0 = time.perf_counter()
        info = h.plan_head_pages(w.qo_indptr, out_ptr_h, w.last_page_len)
        plan_times.append(time.perf_counter() - t0)
    plan_us = float(np.median(plan_times) * 1e6)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        lib.quest_select(q, kmin, kmax, kvp, kvi, budget, out_ptr, n_max, out_indices=out_idx, scores=scores)
        h.run(q, k, v, out_idx, o, lse)

    times, wall = timed_steps(step, steps, warmup, stream, flush, mode)
    h.check()
    med = float(np.median(times))
    n_pages = int(np.diff(w.kv_indptr.astype(np.int64)).sum())
    kept = int(out_ptr_h[-1])
    kept_keys = 0
    for r in range(w.batch):
        n = int(w.kv_indptr[r + 1] - w.kv_indptr[r])
        kept_keys += (min(n, budget) - 1) * w.page_size + int(w.last_page_len[r]) if n else 0
    elt = 2
    summary_bytes = 2 * n_pages * w.num_kv_heads * w.head_dim * elt
    kv_bytes = 2 * kept_keys * w.num_kv_heads * w.head_dim * elt
    qo_bytes = 2 * w.batch * w.num_qo_heads * w.head_dim * elt + 4 * w.batch * w.num_qo_heads
    work_bytes = summary_bytes + kv_bytes + qo_bytes + 4 * (n_pages + kept)
    gbs = work_bytes / (med * 1e-3) / 1e9
    out = dict(workload=name, dtype=w.dtype, page_budget=budget, bytes=work_bytes, summary_bytes=summary_bytes,
               kv_bytes=kv_bytes, ms_median=med, ms_min=float(times.min()), wall_s=wall, plan_us=plan_us,
               plan=info, hbm_GBps=gbs, hbm_frac=gbs / HBM_PEAK_GBS,
               roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=round(gbs / HBM_PEAK_GBS, 4), traffic=None))
    if graph:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(stream)
            with torch.cuda.stream(s):
                step()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step()
            gt, _ = timed_steps(g.replay, steps, warmup, stream, flush, mode)
            out["graph_ms_median"] = float(np.median(gt))
        except Exception as exc:  # report, do not hide
            out["graph_error"] = repr(exc)
    return out, None


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if not readable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, budget_s=10.0):
    """The oracle as it stands, on the full workload, repeated for about budget_s."""
    import threadpoolctl

    import oracle

    cores = len(os.sched_getaffinity(0))
    q = w.q.double().numpy()
    k = w.k_pool.float().numpy()
    v = w.v_pool.float().numpy()
    reps = 0
    t0 = time.perf_counter()
    with threadpoolctl.threadpool_limits(limits=cores):
        while True:
            oracle.bsr_attention(
                q, k, v, w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, w.page_size,
                w.num_qo_heads, w.num_kv_heads, w.scale, w.causal, w.cap, w.window,
            )
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = (time.perf_counter() - t0) / reps
    work = algorithmic_work(w)
    return dict(
        value=work["bytes"] / dt / 1e12,
        unit="TB/s",
        cores=cores,
        cpu_model=cpu_model(),
        kind="oracle",
        sample=f"whole {w.name} workload ({w.batch} requests, all heads), {reps} repetition(s), {dt:.2f} s each",
        seconds_per_step=dt,
    )


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default=",".join(ALL))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--num-workgroups", type=int, default=0, help="persistent grid (0: device resident count)")
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read")
    ap.add_argument("--static-queues", action="store_true",
                    help="run every work item on the workgroup the plan assigns (no run-time claiming)")
    ap.add_argument("--no-headline", action="store_true",
                    help="run only --workloads (for profiling one kernel); prints their results only")
    args = ap.parse_args()
    global STATIC_QUEUES
    STATIC_QUEUES = args.static_queues
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device="cuda:0") if args.flush_mib > 0 else None
    names = [n for n in args.workloads.split(",") if n]
    if HEADLINE not in names and not args.no_headline:
        names = [HEADLINE] + names
    results = {}
    keep = {}
    for name in names:
        if name in APPEND:
            r, ctx = bench_append(name, args.steps, args.warmup, flush, mode=args.flush)
        elif name in QUEST:
            r, ctx = bench_quest(name, args.steps, args.warmup, flush, mode=args.flush, graph=not args.no_graph)
        else:
            r, ctx = bench_workload(name, args.steps, args.warmup, flush, graph=not args.no_graph,
                                    nwg=args.num_workgroups, mode=args.flush)
        results[name] = r
        print(f"[bench] {name}: {json.dumps({k: v for k, v in r.items() if k != 'plan'})}", file=sys.stderr, flush=True)
        if name == HEADLINE:
            keep[name] = ctx
        else:
            del ctx
            torch.cuda.empty_cache()
    if args.no_headline:
        print(json.dumps({"workloads": {n: {k: v for k, v in r.items() if k != "plan"} for n, r in results.items()}}))
        return
    head = results[HEADLINE]
    if "error" in head:
        raise RuntimeError(head["error"])
    ms = head["ms_median"]
    gbs = head["hbm_GBps"]
    prof = torch.cuda.get_device_properties(0)
    line = {
        "metric": METRIC,
        "value": round(gbs / 1000.0, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": {
            "workload": HEADLINE,
            "batch": 64,
            "qo_len": 1,
            "kv_len": "uniform[512,8192]",
            "page_size": 16,
            "heads": "32q/8kv",
            "head_dim": 128,
        },
        # dominant kernel: the persistent kernel of the headline workload, timed per
        # launch with HIP events on its own stream
        "roofline": head["roofline"],
        "device": {"name": prof.name, "arch": getattr(prof, "gcnArchName", ""), "cus": prof.multi_processor_count},
        "workloads": {
            n: {k: v for k, v in r.items() if k not in ("plan",)} | ({"plan": r["plan"]} if "plan" in r else {})
            for n, r in results.items()
        },
    }
    if not args.no_cpu_baseline:
        w, _h = keep[HEADLINE]
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
