"""Algorithmic byte counts of one fused selection call (host-side, from bounds).

Per row with live length L, nlb = ceil(L / B) live blocks:

* reads   ``4 * L`` when the values can change the result, i.e. when some block
          must be dropped (``nlb > K_blk``) or some column must be dropped
          (``L > K_tok``), or when block scores are requested; otherwise every
          live block and column is kept and the outputs follow from the bounds;
* stores  ``4 * B * max(nlb - K_blk, 0)`` bytes of -inf (only the newest block
          can be partial, and it is always kept), when the mask is written;
* stores  ``4 * (K_blk + K_tok)`` bytes of indices, padding included, plus
          ``4 * nlb`` of scores when requested;
* reads   the row's bounds: 4 bytes of end, 4 of start when starts are given.

Workspace traffic (block keys, histograms, lists) is an intermediate and is not
counted.

``plain_bytes`` is the simpler count that charges the ``4 * L`` read on every
non-empty row and 8 bytes of bounds per row, whether or not the values can
change the result.  It is the figure the roofline fraction is quoted on.
"""
from __future__ import annotations

import hashlib
import os

import numpy as np

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


# The sources of the decode-path kernels the counter profiles are taken on.
DECODE_SOURCES = ("dsa_bs_unit.hip", "dsa_device.hpp", "dsa_kernels.hpp", "dsa_select.hip")


def source_sha() -> str:
    """Short hash of the decode-path kernel sources (ties a counter profile to the code)."""
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def row_lengths(starts, ends, rows: int, width: int, starts_repeat: int = 1,
                ends_repeat: int = 1) -> np.ndarray:
    r = np.arange(rows)
    e = np.minimum(np.asarray(ends, dtype=np.int64)[r // ends_repeat], width)
    if starts is None:
        s = np.zeros(rows, dtype=np.int64)
    else:
        s = np.asarray(starts, dtype=np.int64)[r // starts_repeat]
    L = np.where(s < 0, 0, np.maximum(e - s, 0))
    return L


def fused_bytes(starts, ends, rows: int, width: int, block_size: int, k_blocks: int,
                k_tokens: int, starts_repeat: int = 1, ends_repeat: int = 1,
                write_mask: bool = True, with_scores: bool = False) -> dict:
    L = row_lengths(starts, ends, rows, width, starts_repeat, ends_repeat)
    nlb = -(-L // block_size)
    need = (nlb > k_blocks) | (L > k_tokens) | with_scores
    reads = int((4 * L * need).sum())
    mask = int((4 * block_size * np.maximum(nlb - k_blocks, 0)).sum()) if write_mask else 0
    idx = rows * 4 * (k_blocks + k_tokens)
    sc = int((4 * nlb).sum()) if with_scores else 0
    bounds = rows * (4 + (4 if starts is not None else 0))
    total = reads + mask + idx + sc + bounds
    return dict(read_bytes=reads + bounds, mask_bytes=mask, index_bytes=idx,
                score_bytes=sc, total_bytes=total, live_columns=int(L.sum()))


def plain_bytes(starts, ends, rows: int, width: int, block_size: int, k_blocks: int,
                k_tokens: int, starts_repeat: int = 1, ends_repeat: int = 1,
                write_mask: bool = True) -> dict:
    """Per call: 4*L read on every row, 4*B*max(nlb - K_blk, 0) of -inf,
    4*(K_blk + K_tok) of indices with pads, and 8 bytes of bounds per row."""
    L = row_lengths(starts, ends, rows, width, starts_repeat, ends_repeat)
    nlb = -(-L // block_size)
    reads = int((4 * L).sum())
    mask = int((4 * block_size * np.maximum(nlb - k_blocks, 0)).sum()) if write_mask else 0
    idx = rows * 4 * (k_blocks + k_tokens)
    bounds = rows * 8
    return dict(read_bytes=reads, mask_bytes=mask, index_bytes=idx, bounds_bytes=bounds,
                total_bytes=reads + mask + idx + bounds, live_columns=int(L.sum()))
