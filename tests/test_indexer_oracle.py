"""Pins of the indexer-logits oracle (CPU only), and mutants they must catch.

The FP8 decoder is pinned to code points that the OCP 8-bit floating point
specification fixes for E4M3 (bias 7, subnormals, 448 as the largest value,
one NaN pattern per sign, no infinities).  The logit formula is pinned by
hand-worked rows: a negative dot product dropped by the ReLU, a negative head
weight, a key scale, and the selection chain on top of hand-computed logits.
"""
import importlib.util
import math
import os

import numpy as np
import pytest

from oracle import indexer_oracle as io
from sparse_attention_indexer_start_amd import workloads as wl

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle",
                           "indexer_oracle.py")

# E4M3 code -> value, as the OCP OFP8 specification defines them.
SPEC_POINTS = [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 0.875 * 2.0 ** -6), (0x08, 2.0 ** -6),
    (0x30, 0.5), (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0), (0x77, 240.0), (0x78, 256.0),
    (0x7E, 448.0), (0xB8, -1.0), (0xC0, -2.0), (0xFE, -448.0), (0x81, -(2.0 ** -9)),
]


def _code(x: float) -> int:
    for c, v in SPEC_POINTS:
        if v == x:
            return c
    raise KeyError(x)


# ---------------------------------------------------------------------------
# Pins (each takes the oracle module under test)
# ---------------------------------------------------------------------------

def pin_e4m3_spec_points(o):
    got = o.e4m3_decode(np.array([c for c, _ in SPEC_POINTS], np.uint8))
    want = np.array([v for _, v in SPEC_POINTS])
    assert np.array_equal(got, want), (got, want)
    assert np.signbit(o.e4m3_decode(np.array([0x80], np.uint8))[0])     # -0
    assert np.isnan(o.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def pin_e4m3_order(o):
    """Codes 0x00..0x7E are the non-negative values in increasing order, and
    the sign bit mirrors them."""
    pos = o.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = o.e4m3_decode(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -pos)


def pin_logits_worked(o):
    """H=2, D=2, three keys.

    q[0] = (1, 2), q[1] = (-1, 0.5); keys (1, 1), (2, -1), (-1, -2);
    w = (0.5, 2); key scales (0.5, 0.5, 1).
    dots, head 0: 3, 0, -5; head 1: -0.5, -2.5, 0   (ReLU: 3, 0, 0 / 0, 0, 0)
    logits: 0.5 * 0.5 * 3 = 0.75;  0.5 * 0 = 0;  1 * 0 = 0.
    """
    q = np.array([[_code(1.0), _code(2.0)], [_code(-1.0), _code(0.5)]], np.uint8)
    k = np.array([[_code(1.0), _code(1.0)], [_code(2.0), _code(-1.0)],
                  [_code(-1.0), _code(-2.0)]], np.uint8)
    w = np.array([0.5, 2.0], np.float32)
    ks = np.array([0.5, 0.5, 1.0], np.float32)
    got = o.indexer_logits_row(q, k, w, ks)
    assert got.dtype == np.float32
    assert got.tolist() == [0.75, 0.0, 0.0], got


def pin_logits_negative_weight(o):
    """A negative head weight subtracts that head's positive score.

    q[0] = (1, 1), q[1] = (2, 0); keys (1, 1), (1, -1);
    dots: head 0: 2, 0; head 1: 2, 2;  w = (1, -0.5);
    logits: 1*2 - 0.5*2 = 1;  1*0 - 0.5*2 = -1 (no key scale).
    """
    q = np.array([[_code(1.0), _code(1.0)], [_code(2.0), _code(0.0)]], np.uint8)
    k = np.array([[_code(1.0), _code(1.0)], [_code(1.0), _code(-1.0)]], np.uint8)
    w = np.array([1.0, -0.5], np.float32)
    got = o.indexer_logits_row(q, k, w, None)
    assert got.tolist() == [1.0, -1.0], got


def pin_logits_subnormal_products(o):
    """Subnormal codes: (2^-9) * (2^-6) = 2^-15 per dimension, D = 2."""
    q = np.array([[0x01, 0x01]], np.uint8)
    k = np.array([[0x08, 0x08]], np.uint8)
    got = o.indexer_logits_row(q, k, np.array([1.0], np.float32), None)
    assert got.tolist() == [2.0 ** -14], got


def pin_selection_on_worked_logits(o):
    """One query, one head, D=1, keys k[c] = c-th value below; w = 1.

    q = 1, so logits are max(0, k[c]): keys (0.5, 2, 1, 1.5, 0.25, 1)
    -> logits (0.5, 2, 1, 1.5, 0.25, 1).  B=2: block maxima 2, 1.5, pinned;
    K_blk=2 keeps blocks 0 and 2; masked row (0.5, 2, -inf, -inf, 0.25, 1);
    K_tok=3: 2, 1, 0.5 -> columns 0, 1, 5.  Start 0, end 6.
    """
    vals = [0.5, 2.0, 1.0, 1.5, 0.25, 1.0]
    codes = {0.5: 0x30, 2.0: 0x40, 1.0: 0x38, 1.5: 0x3C, 0.25: 0x28}
    k8 = np.array([[codes[v]] for v in vals], np.uint8)
    q8 = np.array([[[0x38]]], np.uint8)
    w = np.array([[1.0]], np.float32)
    bl, tk, lg = o.indexer_select(q8, k8, w, None, None, np.array([6], np.int32), 2, 2, 3,
                                  return_logits=True)
    assert lg[0].tolist() == vals
    assert bl.tolist() == [[0, 2]] and tk.tolist() == [[0, 1, 5]], (bl, tk)


def pin_exact_recipe(o):
    """The synthetic inputs keep every partial sum over heads exact in fp32."""
    case = wl.make_indexer_custom(6, 2048, 64, 128, 8, 16, 64, [2048] * 6, seed=7)
    for t in range(case.queries):
        m = o.exact_fp32_margin(case.q8[t], case.k8, case.w[t], -14)
        assert m < 1.0, m


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(io)


# ---------------------------------------------------------------------------
# Mutants: one planted mistake each in a fresh copy of the oracle
# ---------------------------------------------------------------------------

def _fresh(tag):
    spec = importlib.util.spec_from_file_location(f"oracle.indexer_mut_{tag}", ORACLE_PATH,
                                                  submodule_search_locations=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    spec.loader.exec_module(mod)
    return mod


def _m_fnuz_bias(o):
    orig = o.e4m3_decode

    def e4m3_decode(codes):
        return orig(codes) / 2.0                  # bias 8 (the FNUZ variant's) instead of 7
    o.e4m3_decode = e4m3_decode


def _m_relu_after_weight(o):
    def indexer_logits_row(q8_row, k8_cols, w_row, kscale_cols=None):
        d = o.e4m3_decode(k8_cols) @ o.e4m3_decode(q8_row).T
        s = np.maximum(d * np.asarray(w_row, np.float64)[None, :], 0.0).sum(1)
        if kscale_cols is not None:
            s = s * kscale_cols
        return s.astype(np.float32)
    o.indexer_logits_row = indexer_logits_row


def _m_no_kscale(o):
    orig = o.indexer_logits_row

    def indexer_logits_row(q8_row, k8_cols, w_row, kscale_cols=None):
        return orig(q8_row, k8_cols, w_row, None)
    o.indexer_logits_row = indexer_logits_row


def _m_subnormal_as_normal(o):
    def e4m3_decode(codes):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        sign = np.where(c & 0x80, -1.0, 1.0)
        e = (c >> 3) & 0xF
        m = c & 0x7
        v = np.ldexp(1.0 + m / 8.0, e - 7) * sign    # E = 0 read as a normal number
        v = np.where(c & 0x7F, v, 0.0 * sign)
        return np.where((e == 15) & (m == 7), np.nan, v)
    o.e4m3_decode = e4m3_decode


def _m_inf_codes(o):
    orig = o.e4m3_decode

    def e4m3_decode(codes):
        v = orig(codes)
        c = np.asarray(codes, dtype=np.uint8)
        return np.where((c & 0x7F) == 0x78, np.copysign(np.inf, v), v)   # E=15,M=0 as inf
    o.e4m3_decode = e4m3_decode


def _m_token_ids_relative(o):
    orig = o.indexer_select

    def indexer_select(*a, **k):
        out = orig(*a, **k)
        bl, tk = out[0], out[1]
        tk = np.where(tk > 0, tk - 1, tk)                   # off by one on the key position
        return (bl, tk) + tuple(out[2:])
    o.indexer_select = indexer_select


MUTANTS = {
    "fnuz_bias": _m_fnuz_bias,
    "relu_after_weight": _m_relu_after_weight,
    "no_kscale": _m_no_kscale,
    "subnormal_as_normal": _m_subnormal_as_normal,
    "e15_m0_as_infinity": _m_inf_codes,
    "token_position_off_by_one": _m_token_ids_relative,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    o = _fresh(name)
    MUTANTS[name](o)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except Exception as exc:
            failed.append((pin.__name__, type(exc).__name__))
    assert failed, f"no pin catches mutant {name}"


def test_recipe_bounds_hold_at_the_prefill_shape():
    """The exactness margin on sampled rows of the prefill-sized inputs."""
    case = wl.make_indexer_config("indexer_small")
    for t in (0, 100, case.queries - 1):
        e = int(case.ends[t])
        m = io.exact_fp32_margin(case.q8[t], case.k8[:e], case.w[t], -14)
        assert m < 1.0, (t, m)
    assert not math.isnan(float(case.w.sum()))
