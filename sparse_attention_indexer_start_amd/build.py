"""Build ``libdsa_select.so`` in-tree for gfx950 with hipcc.

Run ``python -m sparse_attention_indexer_start_amd.build`` (or call
:func:`build`).  hipcc cross-compiles without a GPU.

The library is linked from twelve objects compiled in parallel: the host unit
(``dsa_select.hip``: the C ABI and the block top-k kernel), the fused FP8
indexer unit (``dsa_indexer.hip``), the cooperative row top-k unit
(``dsa_row_topk.hip``), the sparse attention unit (``dsa_sparse_attn.hip``)
and one unit per specialised block size (``dsa_bs_unit.hip`` with
``-DDSA_BS=<size>``, 0 being the generic code for every other size).  Objects go to ``_build/`` beside the
sources' package.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libdsa_select.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

HOST_SOURCE = os.path.join(CSRC, "dsa_select.hip")
BS_SOURCE = os.path.join(CSRC, "dsa_bs_unit.hip")
INDEXER_SOURCE = os.path.join(CSRC, "dsa_indexer.hip")
ROW_TOPK_SOURCE = os.path.join(CSRC, "dsa_row_topk.hip")
ATTN_SOURCE = os.path.join(CSRC, "dsa_sparse_attn.hip")
BLOCK_SIZES = (0, 1, 2, 4, 8, 16, 32, 64)
SOURCES = [HOST_SOURCE, BS_SOURCE, INDEXER_SOURCE, ROW_TOPK_SOURCE, ATTN_SOURCE]
HEADERS = [os.path.join(CSRC, "dsa_device.hpp"), os.path.join(CSRC, "dsa_kernels.hpp"),
           os.path.join(INCLUDE, "dsa_select.h"), os.path.join(INCLUDE, "dsa_indexer.h"),
           os.path.join(INCLUDE, "dsa_row_topk.h"), os.path.join(INCLUDE, "dsa_sparse_attn.h")]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _common() -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # Packed fp32 vector ops are kept out of generated code on this target.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def units(extra=()) -> list:
    """(object path, compile command) of every translation unit."""
    out = [(os.path.join(BUILD_DIR, "dsa_select.o"),
            [*_common(), *extra, "-c", HOST_SOURCE]),
           (os.path.join(BUILD_DIR, "dsa_indexer.o"),
            # matrix-core results straight into VGPRs (no accumulator copies)
            [*_common(), *extra, "-mllvm", "-amdgpu-mfma-vgpr-form", "-c", INDEXER_SOURCE]),
           (os.path.join(BUILD_DIR, "dsa_row_topk.o"),
            [*_common(), *extra, "-c", ROW_TOPK_SOURCE]),
           (os.path.join(BUILD_DIR, "dsa_sparse_attn.o"),
            [*_common(), *extra, "-c", ATTN_SOURCE])]
    for bs in BLOCK_SIZES:
        out.append((os.path.join(BUILD_DIR, f"dsa_bs{bs}.o"),
                    [*_common(), *extra, f"-DDSA_BS={bs}", "-c", BS_SOURCE]))
    return [(o, cmd + ["-o", o]) for o, cmd in out]


def link_cmd(objs, out: str = LIB_PATH) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]


def _jobs() -> int:
    for var in ("MAX_JOBS", "CMAKE_BUILD_PARALLEL_LEVEL"):
        v = os.environ.get(var, "")
        if v.isdigit() and int(v) > 0:
            return int(v)
    return max(1, min(len(BLOCK_SIZES) + 1, os.cpu_count() or 1))


def _run(cmd) -> subprocess.CompletedProcess:
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False, extra=()) -> str:
    """Compile the library (always recompiles) and return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = units(extra)
    if verbose:
        for _, cmd in jobs:
            print(" ".join(cmd), flush=True)
    with ThreadPoolExecutor(max_workers=_jobs()) as pool:
        results = list(pool.map(_run, [cmd for _, cmd in jobs]))
    for (obj, _), res in zip(jobs, results):
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(obj)} ({res.returncode}):\n"
                               f"{res.stderr[-8000:]}")
        if verbose and res.stderr.strip():
            print(res.stderr[-4000:], file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    res = _run(link_cmd([o for o, _ in jobs], tmp))
    if res.returncode != 0:
        raise RuntimeError(f"link failed ({res.returncode}):\n{res.stderr[-8000:]}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
