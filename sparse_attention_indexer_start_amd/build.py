"""Build ``libdsa_select.so`` in-tree for gfx950 with hipcc.

Run ``python -m sparse_attention_indexer_start_amd.build`` (or call
:func:`build`).  hipcc cross-compiles without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libdsa_select.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "dsa_select.hip")]
HEADERS = [os.path.join(CSRC, "dsa_device.hpp"), os.path.join(INCLUDE, "dsa_select.h")]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def compile_cmd(out: str = LIB_PATH, extra=()) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        # Packed fp32 vector ops are kept out of generated code on this target.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
        *extra, *SOURCES, "-o", out,
    ]


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles) and return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = compile_cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-8000:]}")
    if verbose and res.stderr.strip():
        print(res.stderr[-4000:], file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
