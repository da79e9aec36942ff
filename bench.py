#!/usr/bin/env python3
"""Benchmark of fused DSA decode-time candidate selection on one MI355X.

One step = one fused selection call (block scores, block top-k, mask, token
top-k) over one batch of seeded synthetic logits already resident in HBM.  The
default workload is the short-context decode batch: fp32 logits [96, 1048576],
block 8, top-256 blocks then top-2048 tokens, ends lognormal(median 400,
sigma 0.8) clipped to [1, 8192].

The timed region is a HIP-graph replay of K steps, each on its own copy of
the input (so every step sees unmasked logits and no step hits another's
cache lines), bracketed by device synchronisation.  Per-call kernel time is
then measured with HIP events around each call on the launch stream, and the
CPU oracle is timed on a bounded sample of the same workload.

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
    """The oracle as it stands, on a bounded sample of the same rows."""
    import numpy as np
    import oracle
    sh = case.shape
    rows = list(range(sh.rows))
    lens = [oracle.row_bounds(r, case.starts, case.ends, sh.width, sh.starts_repeat,
                              sh.ends_repeat)[2] for r in rows]
    # Longest rows first would bias the sample; walk rows in order.
    done = 0
    t0 = time.perf_counter()
    passes = 0
    while True:
        for r in rows:
            s, e, L = oracle.row_bounds(r, case.starts, case.ends, sh.width,
                                        sh.starts_repeat, sh.ends_repeat)
            if L:
                live = np.array(case.logits[r, s:e], dtype=np.float32)
                oracle.select_row(live, sh.block_size, sh.k_blocks, sh.k_tokens)
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        else:
            passes += 1
            continue
        break
    dt = time.perf_counter() - t0
    return dict(value=done / dt, unit="rows/s", cores=1, kind="oracle",
                sample=f"{done} rows of the workload in order ({passes} full passes), "
                       f"{dt:.1f} s on 1 host thread (numpy)",
                live_columns_per_row_mean=float(np.mean(lens)))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="short_decode",
                    choices=["tiny", "short_decode", "mtp_ragged", "long_decode", "prefill_chunk"])
    ap.add_argument("--no-graph", action="store_true", help="time eager calls instead")
    ap.add_argument("--no-mask", action="store_true", help="do not write the mask")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--buffer-budget-gb", type=float, default=48.0)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the selection has no multi-GPU path here.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from sparse_attention_indexer_start_amd import binding, metrics
    from sparse_attention_indexer_start_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    binding.load()
    dev = torch.device("cuda", 0)

    log(f"generating {args.workload}")
    case = wl.make_config(args.workload)
    sh = case.shape
    write_mask = not args.no_mask
    nbytes = case.buf.nbytes
    need = args.steps + args.warmup
    nbuf = int(max(1, min(need, (args.buffer_budget_gb * 2**30) // nbytes)))
    log(f"{nbuf} device copies of {nbytes / 2**20:.1f} MiB ({nbytes} bytes each)")
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

    log("warmup")
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    restore(range(args.warmup))
    torch.cuda.synchronize()

    steps = args.steps
    first = args.warmup
    use_graph = not args.no_graph
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

    log(f"timed region: {steps} steps ({'graph replay' if use_graph else 'eager'})")
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
    log(f"timed region {region_ms:.3f} ms (wall {wall * 1e3:.3f} ms)")

    # Per-call kernel time: HIP events around each call on the launch stream.
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
    call_ms = float(np.mean(durs))

    alg = metrics.fused_bytes(case.starts, case.ends, sh.rows, sh.width, sh.block_size,
                              sh.k_blocks, sh.k_tokens, sh.starts_repeat, sh.ends_repeat,
                              write_mask=write_mask)
    per_call = alg["total_bytes"]
    ms_per_step = region_ms / steps
    value = sh.rows * steps / (region_ms * 1e-3)
    live_gbps = per_call / (ms_per_step * 1e-3) / 1e9
    achieved = per_call / (call_ms * 1e-3) / 1e9
    sha = metrics.source_sha()
    traffic = measured_traffic(args.workload, sha)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline(case, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "rows": sh.rows, "width": sh.width,
            "block_size": sh.block_size, "k_blocks": sh.k_blocks, "k_tokens": sh.k_tokens,
            "col_stride": cs, "write_mask": write_mask, "graph": use_graph,
            "distinct_buffers": nbuf, "programs_per_row": info.programs_per_row,
            "threads_per_group": info.threads_per_group,
            "launches_per_call": info.fused_launches,
        },
        "live_bytes_per_step": per_call,
        "live_GBps": live_gbps,
        "pct_of_hbm_peak": 100.0 * live_gbps / HBM_PEAK_GBPS,
        "kernel_ms_per_call": call_ms,
        "kernel_ms_p10_p90": [float(np.percentile(durs, 10)), float(np.percentile(durs, 90))],
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "source_sha": sha,
        "buffer_bytes": nbytes,
    }
    print(json.dumps(out), flush=True)
    ctx.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
