"""Plant one plausible mistake in a copy of the oracle; some pin must fail.

Every mutant is built on the CPU from a fresh copy of ``oracle/dsa_oracle.py``
with one function replaced, so the other functions of that copy call the
mutated one.  The real oracle is never modified.
"""
import importlib.util
import os

import numpy as np
import pytest

from tests import oracle_pins

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "dsa_oracle.py")


def _fresh_copy(tag):
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{tag}", ORACLE_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _m_tie_high(o):
    def top_k_indices(keys, k):
        keys = np.asarray(keys, dtype=np.uint32)
        k = min(int(k), keys.size)
        idx = np.arange(keys.size, dtype=np.int64)
        order = np.lexsort((-idx, -keys.astype(np.int64)))      # ties to the HIGHER index
        return np.sort(order[:k])
    o.top_k_indices = top_k_indices


def _m_smallest(o):
    def top_k_indices(keys, k):
        keys = np.asarray(keys, dtype=np.uint32)
        k = min(int(k), keys.size)
        idx = np.arange(keys.size, dtype=np.int64)
        order = np.lexsort((idx, keys.astype(np.int64)))        # smallest instead of largest
        return np.sort(order[:k])
    o.top_k_indices = top_k_indices


def _m_key_sign(o):
    def order_keys(values):
        u = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)
        return (u ^ np.uint32(0x80000000)).astype(np.uint32)   # forgets to invert negatives
    o.order_keys = order_keys


def _m_no_pin(o):
    orig = o.block_scores_live

    def block_scores_live(vals, B):
        sc = orig(vals, B)
        if sc.size:
            L = vals.size
            last = vals[(sc.size - 1) * B:L]
            sc[-1] = last[np.argmax(o.order_keys(last))]        # newest block not pinned
        return sc
    o.block_scores_live = block_scores_live


def _m_pin_first(o):
    orig = o.block_scores_live

    def block_scores_live(vals, B):
        sc = orig(vals, B)
        if sc.size > 1:
            L = vals.size
            last = vals[(sc.size - 1) * B:L]
            sc[-1] = last[np.argmax(o.order_keys(last))]
            sc[0] = np.inf                                      # pins the oldest block
        return sc
    o.block_scores_live = block_scores_live


def _m_score_first_elem(o):
    def block_scores_live(vals, B):
        L = vals.size
        nlb = o.num_live_blocks(L, B)
        sc = np.array([vals[b * B] for b in range(nlb)], dtype=np.float32)  # first, not max
        if nlb:
            sc[-1] = np.inf
        return sc
    o.block_scores_live = block_scores_live


def _m_ignore_start(o):
    orig = o.row_bounds

    def row_bounds(row, starts, ends, width, starts_repeat=1, ends_repeat=1):
        s, e, L = orig(row, None, ends, width, starts_repeat, ends_repeat)
        return s, e, L                                          # every row starts at 0
    o.row_bounds = row_bounds


def _m_no_clamp(o):
    def row_bounds(row, starts, ends, width, starts_repeat=1, ends_repeat=1):
        s = 0 if starts is None else int(starts[row // starts_repeat])
        e = int(ends[row // ends_repeat])                     # end not clamped to width
        return s, e, max(0, e - s)
    o.row_bounds = row_bounds


def _m_no_fill(o):
    def select_tokens_live(masked, k_tokens):
        keys = o.order_keys(masked)
        finite = np.nonzero(keys != np.uint32(0x007FFFFF))[0]  # candidates only
        sub = o.top_k_indices(keys[finite], k_tokens)
        return finite[sub]
    o.select_tokens_live = select_tokens_live


def _m_mask_off_by_one(o):
    orig = o.mask_live

    def mask_live(vals, B, kept_blocks):
        out = orig(vals, B, kept_blocks)
        kb = set(int(b) for b in kept_blocks if b >= 0)
        for b in range(o.num_live_blocks(vals.size, B)):
            if b not in kb and (b + 1) * B < vals.size:
                out[(b + 1) * B] = vals[(b + 1) * B]            # leaves the next column alone
        return out
    o.mask_live = mask_live


def _m_relative_tokens(o):
    orig = o.select_fused

    def select_fused(logits, starts, ends, B, kb, kt, write_mask=True,
                     starts_repeat=1, ends_repeat=1, rows=None):
        bl, tk, sc, mk = orig(logits, starts, ends, B, kb, kt, write_mask,
                              starts_repeat, ends_repeat, rows)
        for r in range(tk.shape[0]):
            s, _, _ = o.row_bounds(r, starts, ends, logits.shape[1], starts_repeat, ends_repeat)
            tk[r][tk[r] >= 0] -= s                              # forgets the + start
        return bl, tk, sc, mk
    o.select_fused = select_fused


def _m_k_off_by_one(o):
    orig = o.select_blocks_live

    def select_blocks_live(scores, k_blocks):
        return orig(scores, k_blocks - 1 if k_blocks > 1 else 1)  # keeps one block too few
    o.select_blocks_live = select_blocks_live


def _m_descending_output(o):
    orig = o.top_k_indices

    def top_k_indices(keys, k):
        return orig(keys, k)[::-1].copy()                       # emits descending ids
    o.top_k_indices = top_k_indices


def _m_repeat_ignored(o):
    def row_bounds(row, starts, ends, width, starts_repeat=1, ends_repeat=1):
        s = 0 if starts is None else int(starts[row])         # indexes by row, not row // repeat
        e = int(ends[row])
        e_c = min(e, width)
        if s < 0:
            return s, e_c, 0
        return s, e_c, max(0, e_c - s)
    o.row_bounds = row_bounds


def _m_negative_id_wraps(o):
    def mask_live(vals, B, kept_blocks):
        out = np.array(vals, dtype=np.float32, copy=True)
        L = out.size
        nlb = o.num_live_blocks(L, B)
        keep = np.zeros(nlb, dtype=bool)
        kb = np.asarray(kept_blocks, dtype=np.int64)
        kb = kb[(kb >= -nlb) & (kb < nlb)]                    # a -1 wraps to the newest block
        keep[kb] = True
        out.view(np.uint32)[~np.repeat(keep, B)[:L]] = o.NEG_INF_BITS
        return out
    o.mask_live = mask_live


MUTANTS = {
    "repeat_ignored": _m_repeat_ignored,
    "negative_id_wraps": _m_negative_id_wraps,
    "tie_to_higher_index": _m_tie_high,
    "selects_smallest": _m_smallest,
    "key_forgets_negatives": _m_key_sign,
    "newest_block_not_pinned": _m_no_pin,
    "pins_oldest_block": _m_pin_first,
    "score_is_first_element": _m_score_first_elem,
    "blocks_from_column_0": _m_ignore_start,
    "end_not_clamped": _m_no_clamp,
    "token_topk_without_fill": _m_no_fill,
    "mask_off_by_one": _m_mask_off_by_one,
    "token_ids_relative": _m_relative_tokens,
    "k_blocks_off_by_one": _m_k_off_by_one,
    "ids_descending": _m_descending_output,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    o = _fresh_copy(name)
    MUTANTS[name](o)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except Exception as exc:   # AssertionError, or a crash the mistake causes
            failed.append((pin.__name__, type(exc).__name__))
    assert failed, f"no pin catches mutant {name}"
