#!/usr/bin/env python3
"""Benchmark of fused DSA decode-time candidate selection on one MI355X.

One step = one fused selection call (block scores, block top-k, mask, token
top-k) over one batch of seeded synthetic logits already resident in HBM.  The
default workload is the short-context decode batch: fp32 logits [96, 1048576],
block 8, top-256 blocks then top-2048 tokens, ends lognormal(median 400,
sigma 0.8) clipped to [1, 8192].

The timed region is a HIP-graph replay of K steps, each on its own copy of
the input (so every step sees unmasked logits and no step hits another's
cache lines), bracketed by device synchronisation and by HIP events on the
launch stream; ms_per_step is the events' time over K.  The roofline
fraction divides the algorithmic bytes of one call (4*L read per row, the
-inf stores, the index stores and 8 bytes of bounds per row) by ms_per_step.
The same run also times the long-decode workload (32 rows x 1M width, the
bandwidth-bound case) under the key "long_decode", the fused FP8 indexer on a
prefill chunk ("indexer_prefill"), the cooperative top-k of 16M-column rows
("row_topk") and the sparse attention over the selected tokens at decode
("sparse_attn": per-row and, for the batch whose rows overlap, union mode),
and the C oracle is timed on all host threads over whole passes of the
default workload.

Prints one JSON line.  ``--gpus`` above 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode selection rows/s + live-byte HBM GB/s (% peak), 96 rows x 1M width"
HBM_PEAK_GBPS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(workload: str, sha: str):
    """HBM bytes per call from committed rocprofv3 counters, if current."""
    path = os.path.join(PROFILE_DIR, f"fused_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != sha:
        return None
    return rec.get("hbm_bytes_per_call")


def cpu_baseline(case, seconds: float):
    """The C oracle as it stands, on all host threads, over whole passes of the
    same workload rows (about ``seconds`` of work)."""
    from oracle import c_oracle
    sh = case.shape
    threads = c_oracle.default_threads()
    c_oracle.load()
    # Calibrate: double the pass count until a call takes a tenth of the budget.
    reps = 1
    while True:
        t0 = time.perf_counter()
        c_oracle.select_case(case, with_scores=False, threads=threads, repeat=reps)
        dt = time.perf_counter() - t0
        if dt >= 0.1 * seconds or reps >= 1 << 20:
            break
        reps *= 2
    reps = int(max(1, min(1 << 24, reps * seconds / max(dt, 1e-6))))
    t0 = time.perf_counter()
    c_oracle.select_case(case, with_scores=False, threads=threads, repeat=reps)
    dt = time.perf_counter() - t0
    return dict(value=sh.rows * reps / dt, unit="rows/s", cores=threads, kind="oracle",
                sample=f"{reps} full passes over the {sh.rows} rows of the workload "
                       f"({sh.rows * reps} rows), {dt:.1f} s on {threads} host threads "
                       f"(C oracle: threshold selection; mask written to a copy)")


def run_workload(name: str, steps: int, warmup: int, write_mask: bool, use_graph: bool,
                 budget_gb: float, width=None) -> dict:
    """Graph replay of `steps` fused calls, each on its own copy of the input."""
    import numpy as np
    import torch
    from sparse_attention_indexer_start_amd import binding, metrics
    from sparse_attention_indexer_start_amd import workloads as wl

    dev = torch.device("cuda", 0)
    log(f"{name}: generating" + (f" at width {width}" if width else ""))
    case = wl.make_config(name, width=width)
    sh = case.shape
    nbytes = case.buf.nbytes
    need = steps + warmup
    nbuf = int(max(1, min(need, (budget_gb * 2**30) // nbytes)))
    log(f"{name}: {nbuf} device copies of {nbytes / 2**20:.1f} MiB")
    base = torch.from_numpy(case.buf).to(dev)
    ring = [base.clone() for _ in range(nbuf)]
    starts = None if case.starts is None else torch.from_numpy(case.starts).to(dev)
    ends = torch.from_numpy(case.ends).to(dev)
    cs = sh.col_stride
    views = [b[:, ::cs] for b in ring]
    ctx = binding.Context(sh.rows, sh.width, sh.block_size, sh.k_blocks, sh.k_tokens,
                          row_stride=sh.row_stride, col_stride=cs,
                          starts_repeat=sh.starts_repeat, ends_repeat=sh.ends_repeat)
    info = ctx.info()
    bids = torch.empty((sh.rows, sh.k_blocks), dtype=torch.int32, device=dev)
    tids = torch.empty((sh.rows, sh.k_tokens), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call(i):
        ctx.select_fused(views[i % nbuf], starts, ends, bids, tids, None, write_mask)

    def restore(idx):
        for i in idx:
            ring[i % nbuf].copy_(base)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    restore(range(warmup))
    torch.cuda.synchronize()

    first = warmup
    graph = None
    if use_graph:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(steps):
                    call(first + i)
            torch.cuda.synchronize()
        except Exception as exc:  # capture unsupported: time eager calls
            log(f"graph capture failed ({exc}); timing eager calls")
            graph, use_graph = None, False
            torch.cuda.synchronize()
            restore(range(first, first + steps))
            torch.cuda.synchronize()

    log(f"{name}: timed region, {steps} steps ({'graph replay' if use_graph else 'eager'})")
    # HIP events on the launch stream bracket the timed region.
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    if use_graph:
        graph.replay()
    else:
        for i in range(steps):
            call(first + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    region_ms = ev0.elapsed_time(ev1)
    status = ctx.read_status()
    if status != 0:
        raise RuntimeError(f"{name}: context status {status:#x} after the timed region")
    log(f"{name}: timed region {region_ms:.3f} ms (wall {wall * 1e3:.3f} ms)")

    # Eager calls with events around each (context only: includes launch gaps).
    restore(range(first, first + steps))
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        call(first + i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    durs = np.array([a.elapsed_time(b) for a, b in evs])   # ms

    args_b = (case.starts, case.ends, sh.rows, sh.width, sh.block_size, sh.k_blocks,
              sh.k_tokens, sh.starts_repeat, sh.ends_repeat)
    plain = metrics.plain_bytes(*args_b, write_mask=write_mask)
    needed = metrics.fused_bytes(*args_b, write_mask=write_mask)
    ms_per_step = region_ms / steps
    per_call = plain["total_bytes"]
    achieved = per_call / (ms_per_step * 1e-3) / 1e9
    sha = metrics.source_sha()
    out = dict(
        workload=name, ms_per_step=ms_per_step, rows_per_s=sh.rows * steps / (region_ms * 1e-3),
        config={
            "workload": name, "rows": sh.rows, "width": sh.width,
            "block_size": sh.block_size, "k_blocks": sh.k_blocks, "k_tokens": sh.k_tokens,
            "col_stride": cs, "starts_repeat": sh.starts_repeat, "ends_repeat": sh.ends_repeat,
            "write_mask": write_mask, "graph": use_graph, "distinct_buffers": nbuf,
            "grid_groups": info.grid_groups, "threads_per_group": info.threads_per_group,
            "launches_per_call": info.fused_launches,
        },
        alg_bytes_per_call=per_call, alg_bytes_breakdown=plain,
        needed_bytes_per_call=needed["total_bytes"],
        eager_call_ms_mean=float(np.mean(durs)),
        eager_call_ms_p10_p90=[float(np.percentile(durs, 10)), float(np.percentile(durs, 90))],
        roofline={
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": measured_traffic(name, sha) if width is None else None,
            "basis": "4*L read + -inf stores + index stores + 8 B bounds per row, per call, "
                     "over the graph replay's time per call (HIP events on the launch stream)",
        },
        source_sha=sha, buffer_bytes=nbytes, case=case,
    )
    ctx.close()
    del ring, views, base
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 matrix peak


def run_indexer(name: str, steps: int, warmup: int) -> dict:
    """Graph replay of `steps` fused FP8 indexer calls (logits never stored)."""
    import numpy as np
    import torch
    from sparse_attention_indexer_start_amd import binding
    from sparse_attention_indexer_start_amd import workloads as wl

    log(f"{name}: generating")
    case = wl.make_indexer_config(name)
    dev = torch.device("cuda", 0)
    d = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q8, k8, w, ks, st, en = d(case.q8), d(case.k8), d(case.w), d(case.kscale), \
        d(case.starts), d(case.ends)
    bids = torch.empty((case.queries, case.k_blocks), dtype=torch.int32, device=dev)
    tids = torch.empty((case.queries, case.k_tokens), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        binding.indexer_select(q8, k8, w, ks, st, en, case.block_size, case.k_blocks,
                               case.k_tokens, case.starts_repeat, case.ends_repeat,
                               block_ids=bids, token_ids=tids)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            call()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    lens = np.minimum(case.ends.astype(np.int64), case.keys)
    live = int(lens.sum())
    # the block pass: 2*H*D flops per (query, live key); kept-column recompute
    # only when K_blk * B > K_tok (not in this configuration)
    flops = 2.0 * case.heads * case.head_dim * live
    achieved = flops / (ms * 1e-3) / 1e12
    return dict(
        ms_per_step=ms, queries_per_s=case.queries / (ms * 1e-3),
        config={"workload": name, "queries": case.queries, "keys": case.keys,
                "heads": case.heads, "head_dim": case.head_dim,
                "block_size": case.block_size, "k_blocks": case.k_blocks,
                "k_tokens": case.k_tokens, "dtype": "fp8 e4m3 in, fp32 accumulate",
                "graph": True},
        flops_per_call=flops, live_keys_per_call=live,
        roofline={"bound": "mfma", "achieved": achieved, "peak": FP8_PEAK_TFLOPS,
                  "unit": "TFLOP/s", "frac": achieved / FP8_PEAK_TFLOPS, "traffic": None,
                  "basis": "2*heads*head_dim flops per (query, live key) over the graph "
                           "replay's time per call"},
    )


def run_row_topk(rows: int, width: int, k: int, steps: int, warmup: int) -> dict:
    """Graph replay of `steps` cooperative row top-k calls over seeded rows."""
    import numpy as np
    import torch
    from sparse_attention_indexer_start_amd import binding, metrics
    from sparse_attention_indexer_start_amd import workloads as wl

    log(f"row top-k {rows} x {width}, k={k}: generating")
    case = wl.make_custom(rows, width, 8, 1, 1, [width] * rows, seed=20261217, dup_frac=0.01)
    dev = torch.device("cuda", 0)
    buf = torch.from_numpy(case.buf).to(dev)
    ends = torch.from_numpy(case.ends).to(dev)
    op = binding.RowTopk(rows, width, k)
    out = torch.empty((rows, k), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        op(buf, None, ends, out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            op(buf, None, ends, out)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    alg = rows * (4 * width + 4 * k + 8)
    achieved = alg / (ms * 1e-3) / 1e9
    pieces = op.pieces()
    op.close()
    return dict(ms_per_step=ms, rows=rows, width=width, k=k, pieces_per_row=pieces,
                alg_bytes_per_call=alg,
                roofline={"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                          "basis": "4*L read + 4*k index stores + 8 B bounds per row over the "
                                   "graph replay's time per call (the row is read twice: the "
                                   "first digit pass, and the second, which also lists the keys "
                                   "from the first digit's bin up; the later passes work on "
                                   "those lists)"})


def attn_device_caches(case):
    """K/V caches of a configuration, drawn on the device: bf16 N(0, 1), or
    E4M3 codes with a random sign, exponent field 3..9 and mantissa."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(int(case.cache_seed))
    shape = (case.num_slots, case.kv_heads, case.head_dim)
    if not case.kv_fp8:
        k = torch.randn(shape, generator=gen, device="cuda", dtype=torch.bfloat16)
        v = torch.randn(shape, generator=gen, device="cuda", dtype=torch.bfloat16)
        return k, v

    def codes():
        c = torch.randint(0, 2, shape, generator=gen, device="cuda", dtype=torch.uint8)
        c.bitwise_left_shift_(7)
        e = torch.randint(3, 10, shape, generator=gen, device="cuda", dtype=torch.uint8)
        c.bitwise_or_(e.bitwise_left_shift_(3))
        del e
        c.bitwise_or_(torch.randint(0, 8, shape, generator=gen, device="cuda", dtype=torch.uint8))
        return c
    return codes(), codes()


def run_attn(name: str, steps: int, warmup: int) -> dict:
    """Graph replay of `steps` sparse-attention calls over a configuration;
    a name ending in ":union" runs it in union mode (each request's rows over
    the union of their ids)."""
    import numpy as np
    import torch
    from sparse_attention_indexer_start_amd import binding
    from sparse_attention_indexer_start_amd import workloads as wl

    base, _, mode = name.partition(":")
    union = mode == "union"
    log(f"{name}: generating")
    case = wl.make_attn_config(base)
    dev = torch.device("cuda", 0)
    kd, vd = attn_device_caches(case)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
        torch.bfloat16).to(dev)
    q, gate = bf(case.q), bf(case.gate)
    ids = torch.from_numpy(case.token_ids).to(dev)
    table = torch.from_numpy(case.page_table).to(dev)
    hq = case.kv_heads * case.group
    out = torch.empty((case.rows, hq, case.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((case.rows, hq), dtype=torch.float32, device=dev)
    op = binding.SparseAttn(case.rows, case.kv_heads, case.group, case.head_dim, case.k_tokens,
                            case.num_slots, rows_per_seq=case.rows_per_seq,
                            page_size=case.page_size, pages_per_seq=case.page_table.shape[1],
                            union_rows=case.rows_per_seq if union else 0)
    stream = torch.cuda.current_stream(dev)

    def call():
        op(q, kd, vd, ids, table, gate, case.sm_scale, out, lse, k_scale=case.k_scale,
           v_scale=case.v_scale)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            call()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    status = op.read_status()
    chunks = op.chunks()
    op.close()
    if status != 0:
        raise RuntimeError(f"{name}: status word {status} after the timed calls")
    n_valid = int((case.token_ids >= 0).sum())
    rps = case.rows_per_seq
    n_union = sum(int(np.unique(g[g >= 0]).size) for g in
                  (case.token_ids[i:i + rps] for i in range(0, case.rows, rps)))
    D = case.head_dim
    elem = 1 if case.kv_fp8 else 2
    gathered = (n_union if union else n_valid) * case.kv_heads * D * elem * 2
    per_row = case.rows * (hq * D * 2 * 3 + case.k_tokens * 4 + hq * 4)
    alg = gathered + per_row
    achieved = alg / (ms * 1e-3) / 1e9
    del kd, vd
    torch.cuda.empty_cache()
    return dict(
        ms_per_step=ms, rows_per_s=case.rows / (ms * 1e-3),
        config={"workload": name, "rows": case.rows, "rows_per_seq": case.rows_per_seq,
                "union_rows": case.rows_per_seq if union else 1,
                "kv_heads": case.kv_heads, "group": case.group, "head_dim": D,
                "k_tokens": case.k_tokens, "page_size": case.page_size, "gate": True,
                "chunks": chunks,
                "dtype": ("fp8 e4m3 K/V, " if case.kv_fp8 else "") + "bf16 in, fp32 accumulate, bf16 out",
                "graph": True},
        attended_tokens_per_call=n_valid, union_tokens_per_call=n_union,
        alg_bytes_per_call=alg,
        roofline={"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                  "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                  "basis": ("K and V rows of every distinct token of each request's rows "
                            "(union mode)" if union else "K and V rows of every attended token")
                           + " (2 * kv_heads * head_dim elements, bf16 or fp8) + q, gate and out "
                           "(bf16) + ids + lse, over the graph replay's time per call; page-table "
                           "reads not counted"},
    )


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="short_decode",
                    choices=["tiny", "short_decode", "mtp_ragged", "long_decode", "prefill_chunk"])
    ap.add_argument("--width", type=int, default=None,
                    help="override the buffer width (same bounds and live values)")
    ap.add_argument("--no-graph", action="store_true", help="time eager calls instead")
    ap.add_argument("--no-mask", action="store_true", help="do not write the mask")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="do not also time the long-decode workload")
    ap.add_argument("--buffer-budget-gb", type=float, default=48.0)
    ap.add_argument("--no-indexer", action="store_true",
                    help="do not also time the fused FP8 indexer (prefill chunk)")
    ap.add_argument("--indexer-only", action="store_true",
                    help="time only the fused FP8 indexer")
    ap.add_argument("--no-row-topk", action="store_true",
                    help="do not also time the cooperative row top-k (16M-column rows)")
    ap.add_argument("--row-topk-only", action="store_true",
                    help="time only the cooperative row top-k")
    ap.add_argument("--no-attn", action="store_true",
                    help="do not also time the sparse attention over the selected tokens")
    ap.add_argument("--attn-only", action="store_true",
                    help="time only the sparse attention")
    ap.add_argument("--attn-workloads",
                    default="attn_decode,attn_decode_fp8,attn_c1,attn_decode_g3,attn_decode_g3:union",
                    help="comma-separated sparse-attention workloads to time")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the selection has no multi-GPU path here.",
              file=sys.stderr)
        return 2

    import torch
    from sparse_attention_indexer_start_amd import binding

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    binding.load()
    write_mask = not args.no_mask
    use_graph = not args.no_graph

    if args.row_topk_only:
        rt = [run_row_topk(1, 16 * 2**20, kk, min(args.steps, 20), min(args.warmup, 2))
              for kk in (2048, 2**20)]
        print(json.dumps({"row_topk": rt}), flush=True)
        return 0
    if args.attn_only:
        at = [run_attn(n, min(args.steps, 20), min(args.warmup, 2))
              for n in args.attn_workloads.split(",")]
        print(json.dumps({"sparse_attn": at}), flush=True)
        return 0
    if args.indexer_only:
        ix = run_indexer("indexer_prefill", min(args.steps, 10), min(args.warmup, 2))
        print(json.dumps({"indexer_prefill": ix}), flush=True)
        return 0
    main_run = run_workload(args.workload, args.steps, args.warmup, write_mask, use_graph,
                            args.buffer_budget_gb, args.width)
    second = None
    if not args.no_secondary and args.workload != "long_decode" and args.width is None:
        second = run_workload("long_decode", args.steps, args.warmup, write_mask, use_graph,
                              args.buffer_budget_gb)
        second.pop("case")

    indexer = None
    if not args.no_indexer and args.width is None:
        indexer = run_indexer("indexer_prefill", min(args.steps, 10), min(args.warmup, 2))

    row_topk = None
    if not args.no_row_topk and args.width is None:
        row_topk = [run_row_topk(1, 16 * 2**20, kk, min(args.steps, 20), min(args.warmup, 2))
                    for kk in (2048, 2**20)]

    attn = None
    if not args.no_attn and args.width is None:
        attn = [run_attn(n, min(args.steps, 20), min(args.warmup, 2))
                for n in args.attn_workloads.split(",")]

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline (C oracle, ~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(main_run["case"], args.cpu_seconds)
    main_run.pop("case")

    out = {
        "metric": METRIC,
        "value": main_run["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_run["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": main_run["config"],
        "live_bytes_per_step": main_run["alg_bytes_per_call"],
        "live_GBps": main_run["roofline"]["achieved"],
        "pct_of_hbm_peak": 100.0 * main_run["roofline"]["frac"],
        "alg_bytes_breakdown": main_run["alg_bytes_breakdown"],
        "needed_bytes_per_call": main_run["needed_bytes_per_call"],
        "eager_call_ms_mean": main_run["eager_call_ms_mean"],
        "eager_call_ms_p10_p90": main_run["eager_call_ms_p10_p90"],
        "roofline": main_run["roofline"],
        "cpu_baseline": cpu,
        "source_sha": main_run["source_sha"],
        "buffer_bytes": main_run["buffer_bytes"],
    }
    if second is not None:
        out["long_decode"] = {k: second[k] for k in (
            "ms_per_step", "rows_per_s", "alg_bytes_per_call", "needed_bytes_per_call",
            "eager_call_ms_mean", "roofline", "config")}
    if indexer is not None:
        out["indexer_prefill"] = indexer
    if row_topk is not None:
        out["row_topk"] = row_topk
    if attn is not None:
        out["sparse_attn"] = attn
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
