"""CPU oracle for DSA decode-time candidate selection.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The library and
its Python binding never call it, and it shares no code with them.

It is a plain, slow statement of what the hot path computes, written from the
pages "DSA candidate-block kernels walk each row's live context" (vllm PR
#57459, Summary) and the report on vllm PR #56628 ("Stride the DSA decode
candidate mask over the live context", sections on implementation and key
source).  Each function names the passage it restates.  Values are only
compared and copied, never rounded, so the arithmetic type is irrelevant:
everything is exact fp32 bit handling.

Readings of the pages that this oracle fixes (they also appear in the design
notes):

* live range: ``e' = min(end, width)``, ``L = max(0, e' - start)``; a row with
  ``L == 0`` or ``start < 0`` selects nothing and writes nothing.
* blocks are counted from ``start``: block ``b`` covers columns
  ``[start + b*B, min(start + (b+1)*B, e'))``; there are ``nlb = ceil(L/B)``.
* block score = the live value with the largest order key, and the block that
  holds column ``e'-1`` (the newest, ``nlb-1``) scores ``+inf``.
* order: the total order of the order-preserving key below (so ``-0 < +0``);
  equal keys go to the lower index.
* block top-k keeps ``min(K_blk, nlb)`` blocks; ids are relative to ``start``,
  ascending, padded with ``-1``.
* the mask writes ``-inf`` to every live column of every block that is not
  kept; no other element of the buffer changes.
* token top-k ranks the masked row over ``[start, e')`` and keeps
  ``min(K_tok, L)`` columns; ids are absolute columns, ascending, padded with
  ``-1``.  When the kept blocks hold fewer columns than that, the remaining
  picks are the lowest-index ``-inf`` columns, which is what ranking the whole
  masked row with ties to the lower index gives.

The pages print no worked input/output pair for this chain, so no pin
compares with printed outputs; every function here is pinned instead by brute
force, closed forms, special cases and invariants in
``tests/test_oracle_pins.py``, and by the cases the pages do print (ragged
ends, sentinels) under ``tests/golden/``.
"""
from __future__ import annotations

import numpy as np

NEG_INF_BITS = np.uint32(0xFF800000)


# ---------------------------------------------------------------------------
# Order key
# ---------------------------------------------------------------------------

def order_keys(values) -> np.ndarray:
    """Map fp32 values to uint32 keys whose unsigned order is the float order.

    Negative floats (sign bit set) are bit-inverted, non-negative ones get the
    sign bit set.  This is the total order used for every comparison: it
    agrees with ``<`` on all non-NaN floats and puts ``-0`` below ``+0``.
    """
    u = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)
    return np.where(u >= np.uint32(0x80000000), ~u, u | np.uint32(0x80000000)).astype(np.uint32)


def top_k_indices(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the ``k`` largest keys, ties to the lower index, ascending.

    A full lexicographic sort on (key descending, index ascending), then the
    first ``k`` indices sorted ascending.
    """
    keys = np.asarray(keys, dtype=np.uint32)
    k = min(int(k), keys.size)
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    idx = np.arange(keys.size, dtype=np.int64)
    order = np.lexsort((idx, -keys.astype(np.int64)))
    return np.sort(order[:k])


# ---------------------------------------------------------------------------
# Row bounds (PR #56628 report, key source: start/end per row via
# row // ROW_REPEAT; PR #57459 Summary: work follows [start, end))
# ---------------------------------------------------------------------------

def row_bounds(row: int, starts, ends, width: int, starts_repeat: int = 1,
               ends_repeat: int = 1):
    """Return ``(s, e_clamped, L)`` for one row.

    ``starts`` may be None (every row starts at column 0).  A negative start is
    outside the contract; the row is then treated as empty (``L = 0``).
    """
    s = 0 if starts is None else int(starts[row // starts_repeat])
    e = int(ends[row // ends_repeat])
    e_c = min(e, width)
    if s < 0:
        return s, e_c, 0
    return s, e_c, max(0, e_c - s)


def num_live_blocks(L: int, B: int) -> int:
    return -(-L // B) if L > 0 else 0


# ---------------------------------------------------------------------------
# Steps on one row's live span (vals = logits[row, s:e'] as fp32)
# ---------------------------------------------------------------------------

def block_scores_live(vals: np.ndarray, B: int) -> np.ndarray:
    """Score of every live block: its max-key value; the newest block is +inf.

    PR #57459 Summary: blocks inside the row's range are scored and the
    newest-block pin keeps its semantics.
    """
    L = vals.size
    nlb = num_live_blocks(L, B)
    if nlb == 0:
        return np.zeros(0, dtype=np.float32)
    keys = np.zeros(nlb * B, dtype=np.uint32)          # 0 is below every key of a float
    keys[:L] = order_keys(vals)
    keys = keys.reshape(nlb, B)
    arg = np.argmax(keys, axis=1)                     # first max; all maxima are the same bits
    padded = np.zeros(nlb * B, dtype=np.float32)
    padded[:L] = vals
    scores = padded.reshape(nlb, B)[np.arange(nlb), arg].copy()
    scores[nlb - 1] = np.float32(np.inf)
    return scores


def select_blocks_live(scores: np.ndarray, k_blocks: int) -> np.ndarray:
    """Top ``min(K_blk, nlb)`` blocks by score, ties to lower id, ascending."""
    return top_k_indices(order_keys(scores), k_blocks)


def mask_live(vals: np.ndarray, B: int, kept_blocks) -> np.ndarray:
    """Copy of the live span with every column of a non-kept block set to -inf.

    PR #56628 report, key source: a column keeps its value only if its block
    (counted from start) is flagged; the others are written -inf.  Only the
    live span is considered here (no writes outside [start, end)).
    """
    out = np.array(vals, dtype=np.float32, copy=True)
    L = out.size
    nlb = num_live_blocks(L, B)
    keep = np.zeros(nlb, dtype=bool)
    kb = np.asarray(kept_blocks, dtype=np.int64)
    kb = kb[(kb >= 0) & (kb < nlb)]
    keep[kb] = True
    col_keep = np.repeat(keep, B)[:L]
    out.view(np.uint32)[~col_keep] = NEG_INF_BITS
    return out


def select_tokens_live(masked: np.ndarray, k_tokens: int) -> np.ndarray:
    """Top ``min(K_tok, L)`` columns of the masked live span (relative ids)."""
    return top_k_indices(order_keys(masked), k_tokens)


def select_row(vals: np.ndarray, B: int, k_blocks: int, k_tokens: int):
    """The whole chain on one row: (scores, block ids, masked span, token ids).

    Order of the steps: block scores, block top-k, candidate mask, token top-k
    (PR #57459: select_candidate_blocks feeds apply_candidate_mask, and the row
    top-k bounds its scan by the same ends).
    """
    scores = block_scores_live(vals, B)
    blocks = select_blocks_live(scores, k_blocks)
    masked = mask_live(vals, B, blocks)
    tokens = select_tokens_live(masked, k_tokens)
    return scores, blocks, masked, tokens


# ---------------------------------------------------------------------------
# Buffer-level operations (the five entry points of the library, restated)
# ---------------------------------------------------------------------------

def _live(logits: np.ndarray, row: int, s: int, e: int) -> np.ndarray:
    return np.array(logits[row, s:e], dtype=np.float32, copy=True)


def block_scores(logits, starts, ends, B, scores, starts_repeat=1, ends_repeat=1):
    """Write ``scores[r, :nlb]`` for each row; other entries are left as they are."""
    rows, width = logits.shape
    out = np.array(scores, dtype=np.float32, copy=True)
    for r in range(rows):
        s, e, L = row_bounds(r, starts, ends, width, starts_repeat, ends_repeat)
        if L == 0:
            continue
        sc = block_scores_live(_live(logits, r, s, e), B)
        out[r, : sc.size] = sc
    return out


def topk_blocks(scores, starts, ends, width, B, k_blocks, starts_repeat=1, ends_repeat=1):
    """Top-k block ids of each row over ``scores[r, :nlb]``, padded with -1."""
    rows = scores.shape[0]
    out = np.full((rows, k_blocks), -1, dtype=np.int32)
    for r in range(rows):
        s, e, L = row_bounds(r, starts, ends, width, starts_repeat, ends_repeat)
        nlb = num_live_blocks(L, B)
        if nlb == 0:
            continue
        ids = select_blocks_live(np.asarray(scores[r, :nlb], dtype=np.float32), k_blocks)
        out[r, : ids.size] = ids
    return out


def candidate_mask(logits, starts, ends, B, block_ids, starts_repeat=1, ends_repeat=1):
    """Return a masked copy of ``logits`` (same shape); -1 / out-of-range ids are ignored."""
    rows, width = logits.shape
    out = np.array(logits, dtype=np.float32, copy=True)
    for r in range(rows):
        s, e, L = row_bounds(r, starts, ends, width, starts_repeat, ends_repeat)
        if L == 0:
            continue
        out[r, s:e] = mask_live(_live(logits, r, s, e), B, block_ids[r])
    return out


def topk_tokens(logits, starts, ends, B, k_tokens, block_ids=None,
                starts_repeat=1, ends_repeat=1):
    """Top-k absolute columns of each row's masked live span, padded with -1.

    With ``block_ids`` the row is ranked as if the mask had been applied for
    those blocks; with None it is ranked as it stands.
    """
    rows, width = logits.shape
    out = np.full((rows, k_tokens), -1, dtype=np.int32)
    for r in range(rows):
        s, e, L = row_bounds(r, starts, ends, width, starts_repeat, ends_repeat)
        if L == 0:
            continue
        vals = _live(logits, r, s, e)
        if block_ids is not None:
            vals = mask_live(vals, B, block_ids[r])
        ids = select_tokens_live(vals, k_tokens)
        out[r, : ids.size] = ids + s
    return out


def select_fused(logits, starts, ends, B, k_blocks, k_tokens, write_mask=True,
                 starts_repeat=1, ends_repeat=1, rows=None):
    """The whole chain per row.

    Returns ``(block_ids [R, K_blk], token_ids [R, K_tok], scores [R, nblocks]
    (NaN where not written), masked logits copy)``.  ``rows`` restricts the work
    to a subset of rows (others stay -1 / unwritten).
    """
    R, width = logits.shape
    nblocks = -(-width // B) if width else 0
    block_ids = np.full((R, k_blocks), -1, dtype=np.int32)
    token_ids = np.full((R, k_tokens), -1, dtype=np.int32)
    scores = np.full((R, nblocks), np.nan, dtype=np.float32)
    masked = np.array(logits, dtype=np.float32, copy=True) if write_mask else None
    for r in (range(R) if rows is None else rows):
        s, e, L = row_bounds(r, starts, ends, width, starts_repeat, ends_repeat)
        if L == 0:
            continue
        sc, bl, mk, tk = select_row(_live(logits, r, s, e), B, k_blocks, k_tokens)
        scores[r, : sc.size] = sc
        block_ids[r, : bl.size] = bl
        token_ids[r, : tk.size] = tk + s
        if write_mask:
            masked[r, s:e] = mk
    return block_ids, token_ids, scores, masked

