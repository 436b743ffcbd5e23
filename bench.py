"""Benchmark of the CSA lightning-indexer top-k on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload s256k] [--no-cpu-baseline]
    python bench.py --sweep        chunk-size and top-k sweeps at S=65,536
    python bench.py --workload attn-s256k [--composite]
                                   sparse attention over 2,048 selected keys per
                                   row at S=262,144 (seeded lists, or with
                                   --composite the indexer's own lists: one step
                                   is then csa_index followed by the attention)

A step is one csa_index call over the whole workload: scoring of every
causally visible (query, compressed key) pair on the matrix cores, the
streaming top-k merge, and the row sort.  Inputs are synthetic, seeded and
already resident in HBM when the timed region starts.  Prints one JSON line.

value       whole-job indexer queries/s = B*S*K / wall time of K steps
roofline    the scoring kernel against the bf16 (or fp8) dense MFMA peak:
            algorithmic flops per launch (2*H*D per visible pair) over the
            kernel's average duration, from HIP events recorded on the
            stream it runs on; `traffic` is the HBM bytes per launch from
            the committed rocprofv3 counter summary when that summary was
            taken on the current kernel source, else null
cpu_baseline the CPU oracle (plain C, fp64) on a seeded sample of rows of
            the same workload, on this host's cores
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "indexer queries/sec + MFMA TFLOP/s (% peak) + peak HBM GB at S=262K, 1 GPU"
PEAK_TFLOPS = {"bf16": 2500.0, "e4m3fn": 5000.0}   # MI355X dense MFMA
KERNEL_SRC = os.path.join(ROOT, "streaming_top_selection_csa_amd", "csrc", "csa_stream.hpp")
PMC_DIR = os.path.join(ROOT, "profiles")
ATTN_SRC = os.path.join(ROOT, "streaming_top_selection_csa_amd", "csrc", "csa_attn.hip")
ATTN_PMC_SUMMARY = os.path.join(ROOT, "profiles", "sparse_attn_s256k_pmc.md")


def visible_pairs(S, T, m, B=1, row_offset=0):
    """Number of (query, key) pairs with key s visible to position t, i.e.
    sum over t in [row_offset, row_offset+S) of min(T, (t+1)//m), in closed
    form: with G(x) = sum_{u=0}^{x} min(T, u//m) the answer is
    G(row_offset+S) - G(row_offset)."""
    def G(x):
        full = m * T - 1            # u >= m*T sees all T keys
        y = min(x, full)
        q, r = divmod(y, m)         # sum_{u=0}^{y} u//m
        tot = m * q * (q - 1) // 2 + q * (r + 1)
        if x > full:
            tot += (x - full) * T
        return tot
    if S <= 0:
        return 0
    return B * (G(row_offset + S) - G(row_offset))


def kernel_sha(src=KERNEL_SRC):
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_from_profile(workload, summary=None, src=KERNEL_SRC):
    """Bytes per launch beyond L2 (HBM and memory-side cache) from a
    committed counter summary, if it was taken on this kernel source and
    workload (profiles/stream_topk_<workload>_pmc.md by default)."""
    if summary is None:
        summary = os.path.join(PMC_DIR, "stream_topk_%s_pmc.md" % workload.replace("-", "_"))
    if not os.path.exists(summary):
        return None
    text = open(summary).read()
    sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    wl = re.search(r"workload:\s*(\S+)", text)
    tb = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (sha and wl and tb) or sha.group(1) != kernel_sha(src) or wl.group(1) != workload:
        return None
    return float(tb.group(1))


def cpu_baseline(inp, wl, nrows, seed=0):
    import numpy as np

    import oracle
    from csa_synth import storage_numpy

    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(wl.S, size=min(nrows, wl.S), replace=False)).astype(np.int64)
    rt = __import__("torch").as_tensor(rows, device=inp["q"].device)
    q = storage_numpy(inp["q"][0].index_select(0, rt))
    w = inp["w"][0].index_select(0, rt).cpu().numpy()
    k = storage_numpy(inp["k"][0])
    qs = inp["q_scale"][0].index_select(0, rt).cpu().numpy() if "q_scale" in inp else None
    ks = inp["k_scale"][0].cpu().numpy() if "k_scale" in inp else None
    threads = min(len(rows), int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1))
    t0 = time.perf_counter()
    pos = rows + wl.row_offset
    oracle.topk_rows(q, w, k, pos, wl.m, wl.k, dtype=wl.dtype, q_scale_rows=qs, k_scale=ks,
                     nthreads=threads)
    dt = time.perf_counter() - t0
    # one thread on every (len/16)-th row of the same sample
    sub = np.arange(0, len(rows), max(1, len(rows) // 16))[:16]
    n1 = len(sub)
    t1 = time.perf_counter()
    oracle.topk_rows(q[sub], w[sub], k, pos[sub], wl.m, wl.k, dtype=wl.dtype,
                     q_scale_rows=qs[sub] if qs is not None else None, k_scale=ks, nthreads=1)
    dt1 = time.perf_counter() - t1
    n_vis = np.minimum(wl.n_keys, (pos + 1) // wl.m)
    return {"value": len(rows) / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "single_thread_value": n1 / dt1,
            "sample": (f"{len(rows)} seeded uniform rows of {wl.name} (mean visible keys "
                       f"{float(n_vis.mean()):.0f}; workload mean {wl.n_keys / 2:.0f}), "
                       f"fp64 scores + full sort, {dt:.1f} s on {threads} threads; "
                       f"single_thread_value from {n1} of them spread over the sample, on "
                       f"one thread (mean visible keys {float(n_vis[sub].mean()):.0f}), "
                       f"{dt1:.1f} s")}


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unavailable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


ATTN_METRIC = "sparse attention over the selected keys, queries/sec, 1 GPU"
COMPOSITE_METRIC = "indexer + sparse attention step, queries/sec, 1 GPU"
INDEXER_FOR = {"attn-s256k": "s256k", "attn-s64k": "s64k", "attn-dec64": "dec64"}


def attn_cpu_baseline(att, aw, nrows, seed=0):
    import numpy as np

    import oracle
    from csa_synth import storage_numpy

    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(aw.S, size=min(nrows, aw.S), replace=False)).astype(np.int64)
    rt = __import__("torch").as_tensor(rows, device=att["q"].device)
    q = storage_numpy(att["q"][0].index_select(0, rt))
    k = storage_numpy(att["k"][0])
    v = storage_numpy(att["v"][0])
    idx = att["idx"][0].index_select(0, rt).cpu().numpy()
    threads = min(len(rows), int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1))
    t0 = time.perf_counter()
    oracle.sparse_attention(q, k, v, idx, aw.softmax_scale, nthreads=threads, with_bound=False)
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} seeded uniform rows of {aw.name}, fp64, {dt:.1f} s"}


def attention(csa, args):
    """Sparse attention at an attention shape; with --composite each step is
    the indexer at the matching shape followed by the attention over its
    lists.  The attention kernel is timed with HIP events on its stream."""
    import torch
    from csa_synth import ATTN_WORKLOADS, WORKLOADS, make_attn_inputs, make_inputs

    aw = ATTN_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    stream = torch.cuda.current_stream(dev)
    att = make_attn_inputs(aw, seed=0, device=dev)
    cpu = None
    if not args.no_cpu_baseline and not args.composite:
        cpu = attn_cpu_baseline(att, aw, 2 * args.cpu_rows)
    ind = None
    if args.composite:
        wl = WORKLOADS[INDEXER_FOR[aw.name]]
        assert (wl.B, wl.S, wl.n_keys, wl.m, wl.k, wl.row_offset) == \
            (aw.B, aw.S, aw.T, aw.m, aw.n_sel, aw.row_offset)
        del att["idx"]  # the indexer's lists replace the seeded ones
        ind = make_inputs(wl, seed=0, device=dev)
        idx = torch.empty((wl.B, wl.S, wl.k), dtype=torch.int32, device=dev)
        score = torch.empty((wl.B, wl.S, wl.k), dtype=torch.float32, device=dev)
        ws = csa.workspace_for(ind["q"], ind["k"], wl.m, wl.k, row_offset=wl.row_offset)
    else:
        idx = att["idx"]
    out = torch.empty((aw.B, aw.S, aw.H, aw.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((aw.B, aw.S, aw.H), dtype=torch.float32, device=dev)
    splits = args.entry_splits
    G, _ = csa.attention_plan(csa.make_attn_desc(aw.B, aw.S, aw.T, aw.H, aw.D, aw.n_sel),
                              csa.make_attn_options(splits))
    aws = csa.attention_workspace_for(att["q"], att["k"], aw.n_sel, splits)
    events = csa.HipEvents(args.steps)

    def step(i=None):
        if ind is not None:
            csa.index(ind["q"], ind["w"], ind["k"], wl.m, wl.k, out_idx=idx, out_score=score,
                      row_offset=wl.row_offset, workspace=ws, stream=stream)
        if i is not None:
            events.record(events.pairs[i][0], stream)
        csa.sparse_attention(att["q"], att["k"], att["v"], idx, aw.softmax_scale, out=out,
                             lse=lse, entry_splits=splits, workspace=aws, stream=stream)
        if i is not None:
            events.record(events.pairs[i][1], stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kernel_ms = [events.elapsed_ms(i) for i in range(args.steps)]
    events.close()
    peak_hbm = torch.cuda.max_memory_allocated(dev)

    entries = int(((idx >= 0) & (idx < aw.T)).sum())       # attended (row, entry) pairs
    flops = 4.0 * aw.H * aw.D * entries                     # q.k and p.v per head
    kernel_avg = sum(kernel_ms) / len(kernel_ms)
    achieved = flops / (kernel_avg * 1e-3) / 1e12
    gathered = entries * 2 * aw.D * 2                        # one key and one value row each
    io = (att["q"].numel() + out.numel() + att["k"].numel() + att["v"].numel()) * 2 + \
        idx.numel() * 4 + lse.numel() * 4
    ms_per_step = 1e3 * elapsed / args.steps
    line = {
        "metric": COMPOSITE_METRIC if ind is not None else ATTN_METRIC,
        "value": aw.B * aw.S * args.steps / elapsed,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": aw.name, "B": aw.B, "S": aw.S, "T": aw.T, "H": aw.H, "D": aw.D,
                   "n_sel": aw.n_sel, "m": aw.m, "row_offset": aw.row_offset,
                   "entry_splits": G,
                   "lists": "indexer" if ind is not None else
                   "seeded", "scale": aw.softmax_scale},
        "attention_kernel_ms": kernel_avg,
        "attended_entries": entries,
        "gathered_gb_per_s": gathered / (kernel_avg * 1e-3) / 1e9,
        "peak_hbm_gb": peak_hbm / 1e9,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": achieved / PEAK_TFLOPS["bf16"],
                     "traffic": traffic_from_profile(aw.name, ATTN_PMC_SUMMARY, ATTN_SRC),
                     "algorithmic_io_gb": io / 1e9,
                     "gathered_gb": gathered / 1e9},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def sweep(csa, args):
    """The S=65,536 workload's five-point sweeps: candidate-log partition
    (chunk_keys), top-k, keys staged per LDS tile (key_tile) and keys per
    key range (the T keys cut into ranges whose exact top-k lists a merge
    pass combines).  Each cell is `warmup` untimed calls and `steps` timed
    ones on resident inputs; scoring_kernel_ms covers the scoring kernel,
    ms_per_step the whole call (with ranges: also the merge and sort)."""
    import torch
    from csa_synth import (CHUNK_SWEEP, KEY_TILE_SWEEP, RANGE_SWEEP, TOPK_SWEEP, WORKLOADS,
                           make_inputs)

    base = WORKLOADS["s64k"]
    dev = torch.device("cuda:0")
    inp = make_inputs(base, seed=0, device=dev)
    cells = [("chunk_keys", dict(chunk_keys=c), base.k) for c in CHUNK_SWEEP] + \
            [("topk", {}, k) for k in TOPK_SWEEP] + \
            [("key_tile", dict(key_tile=t), base.k) for t in KEY_TILE_SWEEP] + \
            [("range_keys", dict(key_splits=base.n_keys // r), base.k) for r in RANGE_SWEEP]
    axes = set(args.sweep_axes.split(",")) if args.sweep_axes else None
    flops = 2.0 * base.H * base.D * visible_pairs(base.S, base.n_keys, base.m, base.B)
    stream = torch.cuda.current_stream(dev)
    for axis, kw, k in cells:
        if axes is not None and axis not in axes:
            continue
        c = kw.get("chunk_keys", 0)
        G = kw.get("key_splits", 0)
        out_idx = torch.empty((base.B, base.S, k), dtype=torch.int32, device=dev)
        out_score = torch.empty((base.B, base.S, k), dtype=torch.float32, device=dev)
        ws = csa.workspace_for(inp["q"], inp["k"], base.m, k, c, key_splits=G)
        info = csa.plan_query(csa.make_desc(base.B, base.S, base.n_keys, base.H, base.D), base.m,
                              k, csa.make_options(chunk_keys=c, num_cus=256, key_splits=G,
                                                  key_tile=kw.get("key_tile", 0)))
        events = csa.HipEvents(args.steps)

        def step(timing=None):
            csa.index(inp["q"], inp["w"], inp["k"], base.m, k, out_idx=out_idx,
                      out_score=out_score, workspace=ws, timing=timing, stream=stream, **kw)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(events.pairs[i])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        kms = sum(events.elapsed_ms(i) for i in range(args.steps)) / args.steps
        events.close()
        print(json.dumps({
            "sweep": axis, "workload": base.name, "S": base.S, "T": base.n_keys,
            "chunk_keys": info.chunk_keys, "k": k, "key_tile": info.keys_per_tile,
            "key_ranges": info.key_splits,
            "range_keys": -(-base.n_keys // info.key_splits), "steps": args.steps,
            "ms_per_step": 1e3 * elapsed / args.steps, "scoring_kernel_ms": kms,
            "queries_per_s": base.B * base.S * args.steps / elapsed,
            "scoring_tflops": flops / (kms * 1e-3) / 1e12,
            "workspace_gb": ws.numel() / 1e9}), flush=True)
        del out_idx, out_score, ws


def grouped(csa, args):
    """The grouped (approximate) indexer on the S=65,536 workload: for each
    query correlation rho (0: the i.i.d. gaussian workload; > 0: q rows of
    one 64-position segment correlated with coefficient rho), group size and
    candidate count, the time of one call and the set recall of its rows
    against the exact path (every row, csa_index) and against the CPU
    oracle (256 sampled rows).  One JSON line per cell."""
    for rho in [float(r) for r in args.grouped_rho.split(",")]:
        grouped_one(csa, args, rho)


def grouped_one(csa, args, rho):
    import numpy as np
    import torch

    import oracle
    from csa_synth import WORKLOADS, make_inputs, sample_rows, storage_numpy

    wl = WORKLOADS["s64k"].with_(q_rho=rho)
    dev = torch.device("cuda:0")
    inp = make_inputs(wl, seed=0, device=dev)
    stream = torch.cuda.current_stream(dev)
    ex_idx, _ = csa.index(inp["q"], inp["w"], inp["k"], wl.m, wl.k)
    rows = sample_rows(wl.S, wl.m, wl.k, n=256)
    o_idx, _ = oracle.topk_rows(storage_numpy(inp["q"][0].index_select(
        0, torch.as_tensor(rows, device=dev))), inp["w"][0].index_select(
        0, torch.as_tensor(rows, device=dev)).cpu().numpy(), storage_numpy(inp["k"][0]), rows,
        wl.m, wl.k)

    def recall(got, want):
        g_valid = got >= 0
        w_valid = want >= 0
        inter = np.array([len(np.intersect1d(a[ga], b[wb], assume_unique=True))
                          for a, ga, b, wb in zip(got, g_valid, want, w_valid)])
        n = w_valid.sum(1)
        r = np.where(n > 0, inter / np.maximum(n, 1), 1.0)
        return float(r.mean()), float(r.min())

    flops_exact = 2.0 * wl.H * wl.D * visible_pairs(wl.S, wl.n_keys, wl.m)
    ex_np = ex_idx[0].cpu().numpy()
    for g in (8, 16, 32, 64):
        for C in (2048, 4096, 8192):
            out_idx = torch.empty_like(ex_idx)
            ws = csa.grouped_workspace_for(inp["q"], inp["k"], wl.m, wl.k, g, C, want_score=False)
            events = csa.HipEvents(args.steps)

            def step(timing=None):
                csa.index_grouped(inp["q"], inp["w"], inp["k"], wl.m, wl.k, g, C,
                                  out_idx=out_idx, want_score=False, workspace=ws, timing=timing,
                                  stream=stream)

            for _ in range(args.warmup):
                step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                step(events.pairs[i])
            torch.cuda.synchronize()
            ms = 1e3 * (time.perf_counter() - t0) / args.steps
            call_ms = sum(events.elapsed_ms(i) for i in range(args.steps)) / args.steps
            events.close()
            got = out_idx[0].cpu().numpy()
            r_all = recall(got, ex_np)
            r_or = recall(got[rows], o_idx)
            print(json.dumps({
                "grouped": True, "workload": wl.name, "S": wl.S, "T": wl.n_keys, "k": wl.k,
                "q_rho": rho, "q_segment": wl.q_seg, "group": g, "candidates": C, "ms_per_step": ms, "call_ms": call_ms,
                "queries_per_s": wl.S / (call_ms * 1e-3),
                "exact_equivalent_tflops": flops_exact / (call_ms * 1e-3) / 1e12,
                "recall_vs_exact_all_rows": {"mean": r_all[0], "min": r_all[1]},
                "recall_vs_oracle_256_rows": {"mean": r_or[0], "min": r_or[1]},
                "workspace_gb": ws.numel() / 1e9}), flush=True)
            del ws, out_idx


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="s256k")
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--key-splits", type=int, default=0,
                    help="key ranges per query block (0 = automatic, 1 = none)")
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--no-score", action="store_true",
                    help="call without a score output (out_score = NULL): indices only")
    ap.add_argument("--key-tile", type=int, default=0,
                    help="keys staged per LDS tile (0 = the library's default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="time the five-point sweeps of the S=65,536 workload (chunk size, "
                         "top-k, staged key tile, key-range size), one JSON line per cell; "
                         "the GPU tests check every cell against the oracle")
    ap.add_argument("--grouped", action="store_true",
                    help="the grouped (approximate) indexer on the S=65,536 workload: time and "
                         "set recall for group sizes 8..64 and 2,048..8,192 candidates")
    ap.add_argument("--grouped-rho", default="0,0.5,0.9",
                    help="with --grouped: comma-separated correlations of q rows within "
                         "64-position segments (0 = the i.i.d. workload)")
    ap.add_argument("--sweep-axes", default="",
                    help="with --sweep: comma-separated subset of chunk_keys,topk,key_tile,"
                         "range_keys")
    ap.add_argument("--entry-splits", type=int, default=0,
                    help="with an attn-* workload: ranges per row of the attention (0 = "
                         "automatic, 1 = none)")
    ap.add_argument("--composite", action="store_true",
                    help="with an attn-* workload: run the indexer before the attention "
                         "each step and attend over its lists")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 times), to scale "
                         "the HBM byte counters of a profiler run")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: measures one GPU only (the indexer path is single-GPU); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import streaming_top_selection_csa_amd as csa
    from csa_synth import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 5}))
        return
    csa.load_library()
    if args.sweep:
        sweep(csa, args)
        return
    if args.grouped:
        grouped(csa, args)
        return
    if args.workload.startswith("attn-"):
        attention(csa, args)
        return
    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    torch.cuda.synchronize()
    free0, total = torch.cuda.mem_get_info(dev)       # hipMemGetInfo
    torch.cuda.reset_peak_memory_stats(dev)
    inp = make_inputs(wl, seed=0, device=dev)
    out_idx = torch.empty((wl.B, wl.S, wl.k), dtype=torch.int32, device=dev)
    want_score = not args.no_score
    out_score = (torch.empty((wl.B, wl.S, wl.k), dtype=torch.float32, device=dev)
                 if want_score else None)
    ws = csa.workspace_for(inp["q"], inp["k"], wl.m, wl.k, args.chunk, wl.row_offset,
                           args.key_splits, want_score=want_score)
    torch.cuda.synchronize()
    in_bytes = sum(t.numel() * t.element_size() for t in inp.values())
    out_bytes = out_idx.numel() * 4 + (out_score.numel() * 4 if want_score else 0)
    ws_bytes = ws.numel()
    events = csa.HipEvents(args.steps)
    stream = torch.cuda.current_stream(dev)
    plan = csa.plan_query(csa.make_desc(wl.B, wl.S, wl.n_keys, wl.H, wl.D, csa.CSA_FP8_E4M3FN
                                        if wl.dtype == "e4m3fn" else csa.CSA_BF16,
                                        1 if wl.dtype == "e4m3fn" else 0,
                                        1 if wl.dtype == "e4m3fn" else 0), wl.m, wl.k,
                          csa.make_options(args.chunk, wl.row_offset,
                                           key_splits=args.key_splits, key_tile=args.key_tile))

    def step(timing=None):
        csa.index(inp["q"], inp["w"], inp["k"], wl.m, wl.k, q_scale=inp.get("q_scale"),
                  k_scale=inp.get("k_scale"), out_idx=out_idx, out_score=out_score,
                  chunk_keys=args.chunk, row_offset=wl.row_offset, key_splits=args.key_splits,
                  workspace=ws, timing=timing, stream=stream, want_score=want_score,
                  key_tile=args.key_tile)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events.pairs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kernel_ms = [events.elapsed_ms(i) for i in range(args.steps)]
    events.close()
    peak_hbm = torch.cuda.max_memory_allocated(dev)
    free1, _ = torch.cuda.mem_get_info(dev)
    device_used = free0 - free1   # what the device lost since the start, torch's cache included

    pairs = visible_pairs(wl.S, wl.n_keys, wl.m, wl.B, wl.row_offset)
    flops = 2.0 * wl.H * wl.D * pairs
    ms_per_step = 1e3 * elapsed / args.steps
    kernel_avg = sum(kernel_ms) / len(kernel_ms)
    peak = PEAK_TFLOPS[wl.dtype]
    achieved = flops / (kernel_avg * 1e-3) / 1e12
    step_tflops = flops / (ms_per_step * 1e-3) / 1e12
    qps = wl.B * wl.S * args.steps / elapsed

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, wl, args.cpu_rows)

    line = {
        "metric": METRIC,
        "value": qps,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype if wl.dtype != "e4m3fn" else "fp8-e4m3",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "S": wl.S, "T": wl.n_keys, "H_I": wl.H,
                   "d_I": wl.D, "m": wl.m, "k": wl.k, "dist": wl.dist,
                   "row_offset": wl.row_offset, "chunk_keys": args.chunk or None,
                   "key_splits": plan.key_splits, "key_tile": plan.keys_per_tile},
        "tflops": step_tflops,
        "mfma_pct_peak": 100.0 * step_tflops / peak,
        "peak_hbm_gb": peak_hbm / 1e9,
        "hbm_breakdown_gb": {"inputs": in_bytes / 1e9, "outputs": out_bytes / 1e9,
                             "workspace": ws_bytes / 1e9},
        "hbm_device_used_gb": device_used / 1e9,
        "scores_returned": want_score,
        "scoring_kernel_ms": kernel_avg,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic_from_profile(wl.name)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
