"""ctypes front of the C oracle (``dsa_oracle_c.c``): threshold selection, all cores.

TEST INFRASTRUCTURE ONLY, like the numpy oracle beside it: only the tests,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

``build()`` compiles ``liboracle_c.so`` next to the source with gcc (plain C99
and pthreads).  ``select(...)`` runs the whole chain on every row of a host
buffer and returns block ids, token ids, scores and the masked buffer.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "dsa_oracle_c.c")
LIB_PATH = os.path.join(HERE, "liboracle_c.so")

_lib = None


def build() -> str:
    """Compile the C oracle (always recompiles); returns the library path."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the C oracle")
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread",
           SOURCE, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C oracle build failed:\n{res.stderr[-4000:]}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.dsa_oracle_select.restype = ctypes.c_int
    lib.dsa_oracle_select.argtypes = [P, P, i64, i64, i64, i64, P, P, i32, i32, i32, i32, i32,
                                      i32, P, P, P, i32, i32]
    _lib = lib
    return lib


def default_threads() -> int:
    """Host threads to use: OMP_NUM_THREADS when set, else every core."""
    v = os.environ.get("OMP_NUM_THREADS", "")
    if v.isdigit() and int(v) > 0:
        return int(v)
    return os.cpu_count() or 1


def _ptr(a):
    return None if a is None else a.ctypes.data


def select(buf: np.ndarray, col_stride: int, width: int, starts, ends, block_size: int,
           k_blocks: int, k_tokens: int, starts_repeat: int = 1, ends_repeat: int = 1,
           write_mask: bool = True, with_scores: bool = True, threads: int = 0,
           repeat: int = 1, out_buf: np.ndarray = None):
    """The chain on every row of the underlying buffer ``buf`` [rows, row_stride].

    Element (r, c) of the view is ``buf[r, c * col_stride]``.  Returns
    ``(block_ids, token_ids, scores or None, masked)`` where ``masked`` is a
    copy of ``buf`` with the mask written (``out_buf`` when given: it must be
    a copy of ``buf`` and is masked in place).  Scores hold NaN where not
    written.
    """
    lib = load()
    buf = np.ascontiguousarray(buf, dtype=np.float32)
    rows = buf.shape[0]
    row_stride = buf.shape[1]
    if width > 0 and rows > 0:
        assert (width - 1) * col_stride < row_stride
    nblocks = -(-width // block_size) if width else 0
    bids = np.empty((rows, k_blocks), np.int32)
    tids = np.empty((rows, k_tokens), np.int32)
    scores = np.full((rows, nblocks), np.nan, np.float32) if with_scores else None
    masked = out_buf if out_buf is not None else buf.copy()
    st = None if starts is None else np.ascontiguousarray(starts, dtype=np.int32)
    en = np.ascontiguousarray(ends, dtype=np.int32)
    n = threads or default_threads()
    rc = lib.dsa_oracle_select(_ptr(buf), _ptr(masked), rows, width, row_stride, col_stride,
                               _ptr(st), _ptr(en), starts_repeat, ends_repeat, block_size,
                               k_blocks, k_tokens, 1 if write_mask else 0, _ptr(bids),
                               _ptr(tids), _ptr(scores), n, repeat)
    if rc != 0:
        raise RuntimeError(f"C oracle failed ({rc})")
    return bids, tids, scores, masked


def select_case(case, write_mask=True, with_scores=True, threads=0, repeat=1, out_buf=None):
    """``select`` on a workload case (``workloads.Case``)."""
    sh = case.shape
    return select(case.buf, sh.col_stride, sh.width, case.starts, case.ends, sh.block_size,
                  sh.k_blocks, sh.k_tokens, sh.starts_repeat, sh.ends_repeat, write_mask,
                  with_scores, threads, repeat, out_buf)
