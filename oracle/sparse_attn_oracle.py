"""CPU oracle of the sparse attention over each query row's selected tokens.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only the tests,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.
It shares no code with the HIP library.

What the pages fix.  The page on vllm PR #57273 ("Qwen4Exp QSA: sm_90 tuning
table", Purpose) describes the consumer of the selection: a split-K kernel
that runs the sparse attention of each query over its 2048 selected tokens,
with grouped query heads (3, 6 or 12 query heads per kv head, 1 or 2 kv
heads, head_dim 256), bf16 (or fp8) K/V in a paged cache, a split-K merge and
a fused output gate, checked against an fp32 reference at rtol = atol = 2e-2.
The page on vllm PR #48726 ("LiteDSA: grouped masked sparse attention")
requires the attention to stay query-exact (each query attends exactly its
own selected set) and reports the log-sum-exp (LSE) beside the output.

Readings taken where the pages print no formula:
  * Attention of query row r, query head h over its selected positions P(r)
    (the row's token ids that are >= 0):
        s_j   = sm_scale * (q[r, h] . K[slot(j), h // G])
        lse   = log sum_j exp(s_j)                  (natural log)
        o     = sum_j exp(s_j - lse) * V[slot(j), h // G]
    with G query heads per kv head, consecutive heads sharing one kv head.
    An empty P(r) gives o = 0 and lse = -inf.
  * Paged cache: position p of sequence n = r // rows_per_seq lives in slot
    table[n, p // page_size] * page_size + p % page_size; without a table the
    slot is p.  Positions whose page is outside the table or unmapped (< 0),
    or whose slot is outside the cache, are skipped and counted as bad.
  * Output gate: o * sigmoid(gate[r, h]) elementwise, when a gate is given.
  * Inputs q, K, V and the gate are bf16 (the upper 16 bits of an IEEE fp32);
    this oracle decodes them exactly and computes in float64.
  * fp8 caches (the page's other K/V format): K and V hold OCP E4M3 codes
    with one scale per tensor, K = e4m3(k) * k_scale and V = e4m3(v) *
    v_scale (decoded by the indexer oracle's pinned E4M3 decoder).
  * A position a row lists more than once is attended once per listing,
    unless ``distinct`` is set: then each row's ids are taken as a set, the
    reading the grouped form of the LiteDSA page needs (it runs one product
    over the union of neighbouring queries' selected positions, each query
    keeping exactly its own set).
"""
from __future__ import annotations

import math

import numpy as np

from .indexer_oracle import e4m3_decode


# ---------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------

def bf16_decode(bits) -> np.ndarray:
    """float64 value of each bf16 code (uint16): sign bit 15, exponent bits
    14..7 with bias 127, mantissa bits 6..0; exponent 0 encodes subnormals
    m/128 * 2^-126, exponent 255 infinities (m = 0) and NaN (m != 0)."""
    c = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(c & 0x8000, -1.0, 1.0)
    e = (c >> 7) & 0xFF
    m = c & 0x7F
    sub = np.ldexp(m / 128.0, -126)
    norm = np.ldexp(1.0 + m / 128.0, np.minimum(e, 254) - 127)
    v = np.where(e == 0, sub, norm)
    v = np.where(e == 255, np.where(m == 0, np.inf, np.nan), v)
    return v * sign


# ---------------------------------------------------------------------------
# Paged cache addressing
# ---------------------------------------------------------------------------

def slot_of(pos: int, seq: int, page_table, page_size: int, num_slots: int) -> int:
    """Cache slot of position ``pos`` of sequence ``seq``, or -1 when it is
    not addressable (negative position, page outside the table or unmapped,
    slot outside the cache)."""
    if pos < 0:
        return -1
    if page_table is None:
        slot = pos
    else:
        page = pos // page_size
        if page >= page_table.shape[1]:
            return -1
        phys = int(page_table[seq, page])
        if phys < 0:
            return -1
        slot = phys * page_size + pos % page_size
    return slot if slot < num_slots else -1


# ---------------------------------------------------------------------------
# Attention of one row
# ---------------------------------------------------------------------------

def attend(q_heads: np.ndarray, keys: np.ndarray, values: np.ndarray, sm_scale: float):
    """Softmax attention of queries [Hg, D] over n keys/values [n, D]
    (float64).  Returns (o [Hg, D], lse [Hg])."""
    hg, d = q_heads.shape
    if keys.shape[0] == 0:
        return np.zeros((hg, d)), np.full(hg, -np.inf)
    s = sm_scale * (q_heads @ keys.T)                 # [Hg, n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    tot = e.sum(axis=1, keepdims=True)
    o = (e @ values) / tot
    lse = (m + np.log(tot))[:, 0]
    return o, lse


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def sparse_attention(q, k_cache, v_cache, token_ids, sm_scale: float, group: int,
                     page_table=None, page_size: int = 1, rows_per_seq: int = 1,
                     gate=None, rows=None, k_scale=None, v_scale=None, distinct=False):
    """Outputs of the sparse attention.

    q: uint16 bf16 [R, Hkv * G, D]; k_cache, v_cache: uint16 bf16
    [num_slots, Hkv, D], or uint8 E4M3 codes with k_scale and v_scale given
    (fp8 caches); token_ids: int32 [R, K] (positions, -1 pads);
    page_table: int32 [num_seqs, pages_per_seq] or None; gate: uint16 bf16
    [R, Hkv * G, D] or None.  ``rows`` limits the work to some rows.
    ``distinct``: a position listed twice in one row is attended once.

    Returns (out float64 [R, Hq, D], lse float64 [R, Hq], bad int64 [R]);
    rows not computed are zero / -inf.
    """
    R, hq, d = q.shape
    num_slots, hkv, _ = k_cache.shape
    assert hq == hkv * group
    fp8 = k_cache.dtype == np.uint8
    assert fp8 == (k_scale is not None) == (v_scale is not None) == (v_cache.dtype == np.uint8)

    def kv(cache, sl, g, scale):
        if not sl.size:
            return np.zeros((0, d))
        if fp8:
            return e4m3_decode(cache[sl, g, :]) * float(scale)
        return bf16_decode(cache[sl, g, :])
    out = np.zeros((R, hq, d))
    lse = np.full((R, hq), -np.inf)
    bad = np.zeros(R, dtype=np.int64)
    for r in (range(R) if rows is None else rows):
        seq = r // rows_per_seq
        slots = []
        seen = set()
        for p in np.asarray(token_ids[r]).tolist():
            if p < 0:
                continue                                  # padding
            if distinct:
                if p in seen:
                    continue                              # listed before
                seen.add(p)
            sl = slot_of(p, seq, page_table, page_size, num_slots)
            if sl < 0:
                bad[r] += 1
                continue
            slots.append(sl)
        slots = np.asarray(slots, dtype=np.int64)
        qd = bf16_decode(q[r])                            # [Hq, D]
        for g in range(hkv):
            kk = kv(k_cache, slots, g, k_scale)
            vv = kv(v_cache, slots, g, v_scale)
            heads = slice(g * group, (g + 1) * group)
            o, ls = attend(qd[heads], kk, vv, sm_scale)
            out[r, heads] = o
            lse[r, heads] = ls
        if gate is not None:
            out[r] = out[r] * sigmoid(bf16_decode(gate[r]))
    return out, lse, bad


def default_scale(head_dim: int) -> float:
    """1 / sqrt(head_dim), the usual softmax scale."""
    return 1.0 / math.sqrt(head_dim)
