"""CPU oracle of the fused indexer-logits producer plus selection.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only the tests,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.
It shares no code with the HIP library.

The page on vllm PR #48726 ("Fused DSA indexer Top-k kernel (LiteTopk)",
Motivation and "LiteTopK: fused indexer scoring and TopK") describes the
prefill indexer as an FP8 multi-query (MQA) score for every query/key pair,
materialised as a [num_q, seq_len] matrix and then reduced by a per-row
top-k; LiteTopK computes the same selection without storing that matrix.
The page names the score but does not print its formula.  The reading taken
here is the published DSA indexer score: per query t with H indexer heads
(one FP8 query vector q[t, h] per head) and one FP8 key vector k[c] per
position shared by all heads,

    logit[t, c] = kscale[c] * sum_h  w[t, h] * max(0, q[t, h] . k[c])

with q and k in the OCP FP8 E4M3 format, w (per query and head) and kscale
(per key) in fp32.  Each row t then goes through the selection chain of the
decode path on its live range [start, end): block scores with the newest
block pinned, top-K_blk blocks, and top-K_tok tokens of the row masked to the
kept blocks (``dsa_oracle.select_row``).  No mask is written: the logits are
never stored.

Precision.  This oracle evaluates the formula in float64 and rounds the
result to float32 once.  For the synthetic inputs of the tests (E4M3 values
with exponent fields 5..7, weights n/16, power-of-two key scales) every dot
product, every weighted term and every partial sum over heads is an exact
multiple of 2^-14 below 2^10 in magnitude, so float64 is exact and any fp32
summation order reaches the same float32 value; ``exact_fp32_margin`` checks
that property on the data itself.
"""
from __future__ import annotations

import numpy as np

from . import dsa_oracle


# ---------------------------------------------------------------------------
# OCP 8-bit floating point, E4M3 variant
# ---------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte as float64 (NaN for the two NaN codes).

    Layout (OCP OFP8 specification): bit 7 sign, bits 6..3 exponent E with
    bias 7, bits 2..0 mantissa M.  E = 0 encodes subnormals M/8 * 2^-6;
    otherwise the value is (1 + M/8) * 2^(E - 7).  E = 15 with M = 7 is NaN;
    there are no infinities, so E = 15 with M < 7 are ordinary values up to
    448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = np.ldexp(m / 8.0, -6)
    norm = np.ldexp(1.0 + m / 8.0, e - 7)
    v = np.where(e == 0, sub, norm) * sign
    return np.where((e == 15) & (m == 7), np.nan, v)


# ---------------------------------------------------------------------------
# Logits of one query row over a range of keys
# ---------------------------------------------------------------------------

def indexer_logits_row(q8_row, k8_cols, w_row, kscale_cols=None) -> np.ndarray:
    """float32 logits of one query over the given keys.

    q8_row: uint8 [H, D]; k8_cols: uint8 [n, D]; w_row: float32 [H];
    kscale_cols: float32 [n] or None (all ones).
    """
    return _logits_decoded(e4m3_decode(q8_row), e4m3_decode(k8_cols), w_row, kscale_cols)


def _logits_decoded(q, k, w_row, kscale_cols):
    """The formula on decoded values: q float64 [H, D], k float64 [n, D]."""
    d = k @ q.T                                   # [n, H]: q[t, h] . k[c]
    w = np.asarray(w_row, dtype=np.float64)
    s = np.maximum(d, 0.0) @ w                    # [n]: sum_h w[h] * max(0, d)
    if kscale_cols is not None:
        s = s * np.asarray(kscale_cols, dtype=np.float64)
    return s.astype(np.float32)


def exact_fp32_margin(q8_row, k8_cols, w_row, unit_log2: int = -14) -> float:
    """max over keys of sum_h |w[h] * max(0, d)| in units of 2^unit_log2,
    divided by 2^24: below 1 means every partial sum of the per-head terms,
    in any order, is an exactly representable float32 when every term is a
    multiple of the unit."""
    q = e4m3_decode(q8_row)
    k = e4m3_decode(k8_cols)
    d = k @ q.T
    terms = np.maximum(d, 0.0) * np.asarray(w_row, dtype=np.float64)[None, :]
    scaled = terms / np.ldexp(1.0, unit_log2)
    if not np.all(scaled == np.round(scaled)):
        return float("inf")                        # a term is not a multiple of the unit
    if scaled.size == 0:
        return 0.0
    return float(np.abs(scaled).sum(axis=1).max() / 2.0 ** 24)


# ---------------------------------------------------------------------------
# The selection on top of the logits
# ---------------------------------------------------------------------------

def indexer_select(q8, k8, w, kscale, starts, ends, B: int, k_blocks: int, k_tokens: int,
                   starts_repeat: int = 1, ends_repeat: int = 1, rows=None,
                   return_logits: bool = False):
    """Block ids [Q, K_blk] (relative to start) and token ids [Q, K_tok]
    (absolute key positions), ascending, padded with -1.

    q8: uint8 [Q, H, D]; k8: uint8 [S, D]; w: float32 [Q, H]; kscale:
    float32 [S] or None; row t reads starts[t // starts_repeat] (None: 0) and
    ends[t // ends_repeat]; the live range is clamped to S.  ``rows`` limits
    the work to some rows (the others stay -1).  With ``return_logits`` a
    dict {row: float32 logits of [start, end')} is returned as well.
    """
    Q = q8.shape[0]
    S = k8.shape[0]
    block_ids = np.full((Q, k_blocks), -1, dtype=np.int32)
    token_ids = np.full((Q, k_tokens), -1, dtype=np.int32)
    logits = {}
    kd = e4m3_decode(k8)                          # every key decoded once
    for t in (range(Q) if rows is None else rows):
        s, e, L = dsa_oracle.row_bounds(t, starts, ends, S, starts_repeat, ends_repeat)
        if L == 0:
            continue
        ks = None if kscale is None else kscale[s:e]
        lg = _logits_decoded(e4m3_decode(q8[t]), kd[s:e], w[t], ks)
        _, bl, _, tk = dsa_oracle.select_row(lg, B, k_blocks, k_tokens)
        block_ids[t, : bl.size] = bl
        token_ids[t, : tk.size] = tk + s
        if return_logits:
            logits[t] = lg
    if return_logits:
        return block_ids, token_ids, logits
    return block_ids, token_ids
