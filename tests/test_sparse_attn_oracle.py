"""Pins of the sparse-attention oracle (CPU only), and mutants they must catch.

The bf16 decoder is pinned to code points fixed by the format (the upper half
of an IEEE binary32) and, over all 65,536 codes, to numpy's own binary32
decoding of the widened bits.  The attention is pinned by hand-worked rows
(one token, two tokens with softmax weights 1/4 and 3/4, equal scores giving
the mean and ln n), a score of 1000 that overflows a softmax without its
maximum subtracted, the head-to-kv-head grouping, hand-computed paged-cache
slots, rows sharing a sequence, the sigmoid gate, skipped padding and
unaddressable ids, and bounds that hold for any softmax average.
"""
import math
import os
import types

import numpy as np
import pytest

from oracle import sparse_attn_oracle as so

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle",
                           "sparse_attn_oracle.py")

BF = {1.0: 0x3F80, -1.0: 0xBF80, 2.0: 0x4000, 0.5: 0x3F00, 3.0: 0x4040, -2.0: 0xC000,
      4.0: 0x4080, 5.0: 0x40A0, 7.0: 0x40E0, 8.0: 0x4100, 0.0: 0x0000, 6.0: 0x40C0}


def _b(vals):
    return np.array([[BF[v] for v in row] for row in vals], dtype=np.uint16)


def _cache(rows_by_slot):
    """[num_slots, 1, D] from a list of per-slot vectors."""
    return _b(rows_by_slot)[:, None, :]


# ---------------------------------------------------------------------------
# Pins (each takes the oracle module under test)
# ---------------------------------------------------------------------------

def pin_bf16_spec_points(o):
    pts = [(0x0000, 0.0), (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0x3F00, 0.5),
           (0x3FC0, 1.5), (0x4049, 3.140625), (0x0001, 2.0 ** -133), (0x0080, 2.0 ** -126),
           (0x007F, 127 / 128 * 2.0 ** -126), (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127),
           (0x7F80, np.inf), (0xFF80, -np.inf)]
    got = o.bf16_decode(np.array([c for c, _ in pts], np.uint16))
    assert got.tolist() == [v for _, v in pts], got
    assert np.signbit(o.bf16_decode(np.array([0x8000], np.uint16))[0])
    assert np.isnan(o.bf16_decode(np.array([0x7FC0, 0xFFC1, 0x7F81], np.uint16))).all()


def pin_bf16_all_codes_widen(o):
    """Every bf16 code is the binary32 whose upper 16 bits it is."""
    codes = np.arange(65536, dtype=np.uint32)
    want = (codes << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = o.bf16_decode(codes.astype(np.uint16))
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_single_token(o):
    """q = (1, 2), k = (3, -1): q.k = 1, scale 0.5 -> lse 0.5, o = v."""
    q = _b([[1.0, 2.0]])[None]
    k = _cache([[3.0, -1.0]])
    v = _cache([[-2.0, 0.5]])
    out, lse, bad = o.sparse_attention(q, k, v, np.array([[0]], np.int32), 0.5, 1)
    assert out[0, 0].tolist() == [-2.0, 0.5] and lse[0, 0] == 0.5 and bad[0] == 0


def pin_two_tokens_worked(o):
    """scale = ln 3, q = (1, 0); k = (0, 5), (1, 7) -> scores 0 and ln 3,
    weights 1/4 and 3/4; v = (4, 0), (0, 8) -> o = (1, 6); lse = ln 4."""
    q = _b([[1.0, 0.0]])[None]
    k = _cache([[0.0, 5.0], [1.0, 7.0]])
    v = _cache([[4.0, 0.0], [0.0, 8.0]])
    out, lse, _ = o.sparse_attention(q, k, v, np.array([[0, 1]], np.int32), math.log(3.0), 1)
    assert np.allclose(out[0, 0], [1.0, 6.0], rtol=0, atol=1e-14), out
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-14


def pin_repeated_ids(o):
    """The two-token case with token 1 listed three times.  Taken as a set
    (distinct) it is the same case: o = (1, 6), lse = ln 4.  Listed three
    times it weighs 3 * 3 against 1: o = (4 / 10, 8 * 9 / 10), lse = ln 10."""
    q = _b([[1.0, 0.0]])[None]
    k = _cache([[0.0, 5.0], [1.0, 7.0]])
    v = _cache([[4.0, 0.0], [0.0, 8.0]])
    ids = np.array([[1, 0, -1, 1, 1]], np.int32)
    out, lse, _ = o.sparse_attention(q, k, v, ids, math.log(3.0), 1, distinct=True)
    assert np.allclose(out[0, 0], [1.0, 6.0], rtol=0, atol=1e-14), out
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-14
    out, lse, _ = o.sparse_attention(q, k, v, ids, math.log(3.0), 1)
    assert np.allclose(out[0, 0], [0.4, 7.2], rtol=0, atol=1e-14), out
    assert abs(lse[0, 0] - math.log(10.0)) < 1e-14


def pin_equal_scores_mean(o):
    """q = 0: every score is 0, o is the mean of the attended values, lse = ln 3
    (the two -1 pads are not attended)."""
    q = _b([[0.0, 0.0]])[None]
    k = _cache([[1.0, 2.0]] * 6)
    v = _cache([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0], [0.5, 0.5], [2.0, -2.0]])
    out, lse, bad = o.sparse_attention(q, k, v, np.array([[3, -1, 0, 5, -1]], np.int32), 1.0, 1)
    assert np.allclose(out[0, 0], [(7 + 1 + 2) / 3, (8 + 2 - 2) / 3], rtol=0, atol=1e-14)
    assert abs(lse[0, 0] - math.log(3.0)) < 1e-14 and bad[0] == 0


def pin_large_scores(o):
    """Two scores of 1000: lse = 1000 + ln 2, o the mean (exp(1000)
    overflows float64 unless the maximum is subtracted)."""
    q = _b([[1.0, 0.0]])[None]
    k = _cache([[1.0, 0.0], [1.0, 0.0]])
    v = _cache([[2.0, 0.0], [0.0, 4.0]])
    out, lse, _ = o.sparse_attention(q, k, v, np.array([[0, 1]], np.int32), 1000.0, 1)
    assert np.allclose(out[0, 0], [1.0, 2.0], rtol=0, atol=1e-14), out
    assert abs(lse[0, 0] - (1000.0 + math.log(2.0))) < 1e-12


def pin_gqa_grouping(o):
    """2 kv heads, 3 query heads each: heads 0-2 read kv head 0, heads 3-5
    kv head 1."""
    q = np.full((1, 6, 2), BF[1.0], np.uint16)
    k = np.full((1, 2, 2), BF[1.0], np.uint16)
    v = np.array([[[BF[1.0], BF[1.0]], [BF[2.0], BF[2.0]]]], np.uint16)
    out, _, _ = o.sparse_attention(q, k, v, np.array([[0]], np.int32), 1.0, 3)
    assert out[0, :, 0].tolist() == [1.0, 1.0, 1.0, 2.0, 2.0, 2.0], out[0, :, 0]


def pin_paged_slots(o):
    """Page size 4, table row (2, 0, 1, -1), 12 slots: position 5 -> page 1
    -> slot 0*4 + 1 = 1; 9 -> slot 1*4 + 1 = 5; 0 -> slot 8; 12 (page 3
    unmapped), 16 (page 4 beyond the table) and -1 -> not addressable.
    Without a table, the slot is the position (12 is beyond 12 slots)."""
    t = np.array([[2, 0, 1, -1]], np.int32)
    got = [o.slot_of(p, 0, t, 4, 12) for p in (5, 9, 0, 3, 12, 16, -1)]
    assert got == [1, 5, 8, 11, -1, -1, -1], got
    assert [o.slot_of(p, 0, None, 4, 12) for p in (7, 11, 12)] == [7, 11, -1]
    vals = [[float(s % 8), 0.0] for s in range(12)]
    v = _cache(vals)
    k = _cache([[0.0, 0.0]] * 12)
    q = _b([[1.0, 1.0]])[None]
    out, _, _ = o.sparse_attention(q, k, v, np.array([[9]], np.int32), 1.0, 1,
                                   page_table=t, page_size=4)
    assert out[0, 0].tolist() == [5.0, 0.0], out


def pin_rows_share_a_sequence(o):
    """Four rows, two per sequence, page size 2: table rows (1, 0) and (0, 1)
    for sequences 0 and 1 (rows 2 and 3 of the table belong to sequences
    that no row reads); position 0 is slot 2 for rows 0-1 and slot 0 for
    rows 2-3."""
    t = np.array([[1, 0], [0, 1], [1, 0], [0, 1]], np.int32)
    v = _cache([[1.0, 0.0], [2.0, 0.0], [3.0, 0.0], [4.0, 0.0]])
    k = _cache([[0.0, 0.0]] * 4)
    q = np.full((4, 1, 2), BF[1.0], np.uint16)
    out, _, _ = o.sparse_attention(q, k, v, np.zeros((4, 1), np.int32), 1.0, 1,
                                   page_table=t, page_size=2, rows_per_seq=2)
    assert out[:, 0, 0].tolist() == [3.0, 3.0, 1.0, 1.0], out[:, 0, 0]


def pin_gate_is_sigmoid(o):
    """Gate 0 halves the output, gate 2 scales it by 1 / (1 + e^-2), gate -inf
    zeroes it."""
    q = _b([[1.0, 1.0]])[None]
    k = _cache([[1.0, 1.0]])
    v = _cache([[4.0, 8.0]])
    g = np.array([[[BF[0.0], BF[2.0]]]], np.uint16)
    out, _, _ = o.sparse_attention(q, k, v, np.array([[0]], np.int32), 1.0, 1, gate=g)
    assert out[0, 0, 0] == 2.0 and abs(out[0, 0, 1] - 8.0 / (1.0 + math.exp(-2.0))) < 1e-14
    g = np.array([[[0xFF80, BF[0.0]]]], np.uint16)
    out, _, _ = o.sparse_attention(q, k, v, np.array([[0]], np.int32), 1.0, 1, gate=g)
    assert out[0, 0].tolist() == [0.0, 4.0]


def pin_unaddressable_ids_skipped(o):
    """Position 100 lies beyond a 2-page table: skipped and counted; the
    result is the attention over positions 0 and 3 alone."""
    t = np.array([[0, 1]], np.int32)
    k = _cache([[0.0, 0.0]] * 4)
    v = _cache([[2.0, 0.0], [5.0, 5.0], [6.0, 6.0], [4.0, 8.0]])
    q = _b([[1.0, 1.0]])[None]
    out, lse, bad = o.sparse_attention(q, k, v, np.array([[0, 100, 3]], np.int32), 1.0, 1,
                                       page_table=t, page_size=2)
    assert out[0, 0].tolist() == [3.0, 4.0] and bad[0] == 1
    assert abs(lse[0, 0] - math.log(2.0)) < 1e-14


def pin_empty_row(o):
    q = _b([[1.0, 1.0]])[None]
    k = _cache([[1.0, 1.0]] * 2)
    v = _cache([[1.0, 1.0]] * 2)
    out, lse, bad = o.sparse_attention(q, k, v, np.full((1, 4), -1, np.int32), 1.0, 1)
    assert out[0, 0].tolist() == [0.0, 0.0] and lse[0, 0] == -np.inf and bad[0] == 0


def pin_softmax_bounds(o):
    """For random rows: max_j s_j <= lse <= max_j s_j + ln n, and each output
    lies within the range of the attended values (a convex combination);
    permuting the ids changes nothing beyond rounding."""
    rng = np.random.default_rng(5)
    S, D, n = 64, 16, 20
    bits = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    k = bits(rng.standard_normal((S, 1, D)))
    v = bits(rng.standard_normal((S, 1, D)))
    q = bits(rng.standard_normal((3, 2, D)))
    ids = np.stack([rng.choice(S, n, replace=False) for _ in range(3)]).astype(np.int32)
    out, lse, _ = o.sparse_attention(q, k, v, ids, 0.25, 2)
    kd, vd, qd = o.bf16_decode(k[:, 0]), o.bf16_decode(v[:, 0]), o.bf16_decode(q)
    for r in range(3):
        for h in range(2):
            s = 0.25 * kd[ids[r]] @ qd[r, h]
            assert s.max() - 1e-12 <= lse[r, h] <= s.max() + math.log(n) + 1e-12
            lo, hi = vd[ids[r]].min(0), vd[ids[r]].max(0)
            assert np.all(out[r, h] >= lo - 1e-12) and np.all(out[r, h] <= hi + 1e-12)
    out2, lse2, _ = o.sparse_attention(q, k, v, ids[:, ::-1].copy(), 0.25, 2)
    assert np.allclose(out, out2, rtol=0, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)


def pin_fp8_cache_scales(o):
    """fp8 caches: E4M3 codes 0x38 = 1, 0x40 = 2, 0x30 = 0.5, 0x44 = 3;
    k_scale 0.5, v_scale 4.  q = (1, 0); keys (2, 1) and (1, 3) -> 2*0.5 = 1
    and 1*0.5 = 0.5; scale ln(3)/0.5 = 2 ln 3 makes the scores ln 9 and
    ln 3: weights 3/4 and 1/4.  V codes (1, 0.5) and (3, 2) times 4 ->
    (4, 2) and (12, 8): o = (3/4*4 + 1/4*12, 3/4*2 + 1/4*8) = (6, 3.5);
    lse = ln(9 + 3) = ln 12."""
    q = _b([[1.0, 0.0]])[None]
    k = np.array([[[0x40, 0x38]], [[0x38, 0x44]]], np.uint8)
    v = np.array([[[0x38, 0x30]], [[0x44, 0x40]]], np.uint8)
    out, lse, _ = o.sparse_attention(q, k, v, np.array([[0, 1]], np.int32), 2.0 * math.log(3.0),
                                     1, k_scale=0.5, v_scale=4.0)
    assert np.allclose(out[0, 0], [6.0, 3.5], rtol=0, atol=1e-13), out
    assert abs(lse[0, 0] - math.log(12.0)) < 1e-13


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(so)


# ---------------------------------------------------------------------------
# Mutants: one planted mistake each, in the oracle's source text
# ---------------------------------------------------------------------------

MUTANTS = {
    "kv_heads_interleaved": ("heads = slice(g * group, (g + 1) * group)",
                             "heads = slice(g, hq, hkv)"),
    "page_offset_dropped": ("slot = phys * page_size + pos % page_size",
                            "slot = phys * page_size"),
    "rows_per_seq_ignored": ("seq = r // rows_per_seq", "seq = r"),
    "pads_wrap": ("            if p < 0:\n                continue",
                  "            if p < 0:\n                p = p % 2"),
    "no_max_subtraction": ("m = s.max(axis=1, keepdims=True)", "m = np.zeros((hg, 1))"),
    "lse_base_two": ("lse = (m + np.log(tot))[:, 0]", "lse = (m + np.log2(tot))[:, 0]"),
    "gate_linear": ("out[r] = out[r] * sigmoid(bf16_decode(gate[r]))",
                    "out[r] = out[r] * bf16_decode(gate[r])"),
    "scale_ignored": ("s = sm_scale * (q_heads @ keys.T)", "s = q_heads @ keys.T"),
    "bf16_bias_126": ("np.minimum(e, 254) - 127)", "np.minimum(e, 254) - 126)"),
    "bf16_subnormal_as_normal": ("sub = np.ldexp(m / 128.0, -126)",
                                 "sub = np.ldexp(1.0 + m / 128.0, -127)"),
    "empty_lse_zero": ("return np.zeros((hg, d)), np.full(hg, -np.inf)",
                       "return np.zeros((hg, d)), np.zeros(hg)"),
    "bad_ids_read_last_slot": ("bad[r] += 1\n                continue", "bad[r] += 1"),
    "distinct_ignored": ("                if p in seen:", "                if False:"),
    "distinct_always": ("            if distinct:\n                if p in seen:",
                        "            if True:\n                if p in seen:"),
    "fp8_scale_ignored": ("return e4m3_decode(cache[sl, g, :]) * float(scale)",
                          "return e4m3_decode(cache[sl, g, :])"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(ORACLE_PATH).read()
    assert src.count(old) == 1, f"mutant {name}: anchor not found once"
    mod = types.ModuleType(f"oracle.sparse_attn_mut_{name}")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(name)
    caught = []
    with np.errstate(all="ignore"):
        for pin in ALL_PINS:
            try:
                pin(mod)
            except Exception:
                caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
