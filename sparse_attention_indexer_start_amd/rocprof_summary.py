"""Summaries of rocprofv3 CSV output for the benchmark's kernels.

    python -m sparse_attention_indexer_start_amd.rocprof_summary kernels DIR OUT.md --cmd "..."
    python -m sparse_attention_indexer_start_amd.rocprof_summary pmc FETCH_DIR WRITE_DIR \
        --workload NAME --copy-bytes N --out OUT.json --cmd "..."

``kernels`` turns ``*_kernel_stats.csv`` into a short markdown table.

``pmc`` reads the per-dispatch ``FETCH_SIZE`` and ``WRITE_SIZE`` counters (KiB)
of two ``--pmc`` runs.  The counters are scaled by what they read for a plain
copy kernel of known size in the same run (the benchmark restores each input
buffer with a device copy of exactly ``--copy-bytes`` bytes), and the scaled
per-call HBM bytes of the selection kernel are written as JSON, together with
the hash of the kernel sources they were taken on.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics

from .metrics import source_sha

KERNEL = "k_fused"
COPY = "__amd_rocclr_copyBuffer"


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def short_name(name: str, limit: int = 120) -> str:
    """Kernel names of library code (torch's templated kernels) cut to a
    readable length."""
    return name if len(name) <= limit else name[:limit] + "..."


def kernel_table(d: str, cmd: str) -> str:
    path = _one(os.path.join(d, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    lines = [f"Command: `{cmd}`", "",
             "| kernel | calls | average us | min us | max us | share % |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    return "\n".join(lines) + "\n"


def _counter(d: str, name: str):
    path = _one(os.path.join(d, "**", "*counter_collection.csv"))
    kern, copy = [], []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != name:
            continue
        v = float(r["Counter_Value"])
        if KERNEL in r["Kernel_Name"]:
            kern.append(v)
        elif r["Kernel_Name"] == COPY:
            copy.append((int(r["Grid_Size"]), v))
    if not kern or not copy:
        raise RuntimeError(f"{name}: no {KERNEL} or {COPY} dispatches in {path}")
    # The buffer restores are the most frequent copy shape.
    grids = [g for g, _ in copy]
    g0 = max(set(grids), key=grids.count)
    cal = statistics.median(v for g, v in copy if g == g0)
    return statistics.median(kern), cal, len(kern)


def pmc_summary(fetch_dir: str, write_dir: str, workload: str, copy_bytes: int,
                cmd_fetch: str, cmd_write: str) -> dict:
    f_k, f_cal, nf = _counter(fetch_dir, "FETCH_SIZE")
    w_k, w_cal, nw = _counter(write_dir, "WRITE_SIZE")
    kib = copy_bytes / 1024.0
    f_scale, w_scale = kib / f_cal, kib / w_cal
    fetch_b = f_k * f_scale * 1024.0
    write_b = w_k * w_scale * 1024.0
    return {
        "workload": workload,
        "source_sha": source_sha(),
        "kernel": KERNEL,
        "dispatches": {"fetch_run": nf, "write_run": nw},
        "fetch_kib_raw_median": f_k,
        "write_kib_raw_median": w_k,
        "copy_bytes": copy_bytes,
        "copy_fetch_kib_raw": f_cal,
        "copy_write_kib_raw": w_cal,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "hbm_fetch_bytes_per_call": fetch_b,
        "hbm_write_bytes_per_call": write_b,
        "hbm_bytes_per_call": fetch_b + write_b,
        "commands": [cmd_fetch, cmd_write],
    }


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("dir")
    k.add_argument("out")
    k.add_argument("--cmd", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("fetch_dir")
    p.add_argument("write_dir")
    p.add_argument("--workload", required=True)
    p.add_argument("--copy-bytes", type=int, required=True)
    p.add_argument("--out", required=True)
    p.add_argument("--cmd-fetch", required=True)
    p.add_argument("--cmd-write", required=True)
    a = ap.parse_args()
    if a.what == "kernels":
        with open(a.out, "w") as f:
            f.write(kernel_table(a.dir, a.cmd))
    else:
        rec = pmc_summary(a.fetch_dir, a.write_dir, a.workload, a.copy_bytes,
                          a.cmd_fetch, a.cmd_write)
        with open(a.out, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))


if __name__ == "__main__":
    main()
