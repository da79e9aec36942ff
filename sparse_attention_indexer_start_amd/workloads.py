"""Seeded synthetic inputs for DSA decode-time candidate selection.

This module only lays out inputs: the fp32 indexer-logits buffer
``[rows, max_model_len]`` (optionally a strided "packed column" view), the
per-row live range ``[start, end)`` and the selection sizes.  It holds none of
the selection arithmetic (no block maxima, no ordering, no masking), so it can
feed both the CPU oracle and the HIP path without coupling them.

Shapes and distributions follow the workloads named for this method:

* ``tiny``          fp32 [4, 4096], block 8, top-64 blocks then top-256 tokens,
                    ends uniform in [1, 4096] with rows 0/1 pinned to 1 and
                    4096, 5% of live values duplicated to force ties.
* ``short_decode``  fp32 [96, 1048576], block 8, top-256 / top-2048, ends from
                    lognormal(median 400, sigma 0.8) clipped to [1, 8192].
                    This stands in for ShareGPT-length decode contexts (a few
                    hundred tokens per request) against a 1M-wide buffer.
* ``mtp_ragged``    [52 requests x 4 rows, 131072] viewed with column stride 2,
                    block 16, top-128 / top-2048, per-request starts uniform in
                    [0, 1024], ends start + U[1, 65536] offset by 0..3 per row,
                    four edge requests with ends 1023/1024/1025/width.
* ``long_decode``   fp32 [32, 1048576], block 8, top-2048 / top-2048, ends
                    uniform in [262144, 1048576], 1% of live values times 8.
* ``prefill_chunk`` fp32 [8192, 131072] = 4 sequences x 2048 queries, causal
                    ends ctx + q + 1 with ctx uniform in [0, 120000], block 8,
                    top-256 / top-2048.

Live values are N(0, 1) fp32 drawn per row from
``numpy.random.default_rng([seed, cfg, row])`` so any single row can be
regenerated on its own.  Columns past ``end`` hold a quiet-NaN sentinel,
columns before ``start`` another, and the interleaved elements of a strided
view a third, so any stray read or write shows up bit-for-bit.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BASE_SEED = 20261202

# Quiet NaNs with distinct payloads (bit patterns), never produced by the path.
SENTINEL_TAIL = np.uint32(0x7FC5A5A5)   # columns at or past end
SENTINEL_HEAD = np.uint32(0x7FC1B1B1)   # columns before start
SENTINEL_GAP = np.uint32(0x7FC3C3C3)    # interleaved elements of a strided view

CONFIG_IDS = {
    "tiny": 1,
    "short_decode": 2,
    "mtp_ragged": 3,
    "long_decode": 4,
    "prefill_chunk": 5,
}


@dataclasses.dataclass
class Shape:
    rows: int
    width: int
    block_size: int
    k_blocks: int
    k_tokens: int
    col_stride: int = 1
    starts_repeat: int = 1
    ends_repeat: int = 1

    @property
    def row_stride(self) -> int:
        return self.width * self.col_stride

    @property
    def nblocks(self) -> int:
        return -(-self.width // self.block_size) if self.width else 0


@dataclasses.dataclass
class Case:
    """One workload instance.

    ``buf`` is the underlying fp32 storage ``[rows, width * col_stride]``;
    ``logits`` is the ``[rows, width]`` view the method operates on.
    ``starts`` is None (all rows start at 0) or int32 indexed by
    ``row // starts_repeat``; ``ends`` is int32 indexed by
    ``row // ends_repeat``.
    """
    name: str
    shape: Shape
    buf: np.ndarray
    starts: Optional[np.ndarray]
    ends: np.ndarray
    seed: int

    @property
    def logits(self) -> np.ndarray:
        return self.buf[:, :: self.shape.col_stride]

    def live_range(self, row: int):
        """(start, end clamped to width) of ``row`` as stored in the inputs."""
        sh = self.shape
        s = 0 if self.starts is None else int(self.starts[row // sh.starts_repeat])
        e = int(self.ends[row // sh.ends_repeat])
        return s, min(e, sh.width)


def _row_rng(seed: int, cfg: int, row: int) -> np.random.Generator:
    return np.random.default_rng([seed, cfg, row])


def _fill_row(buf_row: np.ndarray, col_stride: int, width: int, s: int, e: int,
              rng: np.random.Generator, block_size: int,
              dup_frac: float = 0.0, outlier_frac: float = 0.0,
              outlier_scale: float = 8.0) -> None:
    """Write one row: head sentinel, N(0,1) live span, tail sentinel, gaps."""
    u = buf_row.view(np.uint32)
    if col_stride > 1:
        u[:] = SENTINEL_GAP
    view = u[::col_stride]
    s_c = max(0, min(s, width))
    e_c = max(s_c, min(e, width))
    view[:s_c] = SENTINEL_HEAD
    view[e_c:] = SENTINEL_TAIL
    n = e_c - s_c
    if n <= 0:
        return
    vals = rng.standard_normal(n, dtype=np.float32)
    if outlier_frac > 0.0:
        m = int(round(outlier_frac * n))
        if m:
            pos = rng.choice(n, size=m, replace=False)
            vals[pos] *= np.float32(outlier_scale)
    if dup_frac > 0.0 and n > 1:
        m = int(round(dup_frac * n))
        # Half as single-value copies between random live positions.
        m1 = m // 2
        if m1:
            src = rng.integers(0, n, size=m1)
            dst = rng.integers(0, n, size=m1)
            vals[dst] = vals[src]
        # Half as whole-block copies (block aligned relative to start), which
        # makes two blocks hold identical values and hence identical scores.
        nfull = n // block_size
        copies = (m - m1) // max(1, block_size)
        if nfull >= 2 and copies:
            src_b = rng.integers(0, nfull, size=copies)
            dst_b = rng.integers(0, nfull, size=copies)
            for a, b in zip(src_b, dst_b):
                vals[b * block_size:(b + 1) * block_size] = \
                    vals[a * block_size:(a + 1) * block_size]
    view[s_c:e_c] = vals.view(np.uint32)


def _alloc(shape: Shape) -> np.ndarray:
    return np.empty((shape.rows, shape.width * shape.col_stride), dtype=np.float32)


def build_case(name: str, shape: Shape, starts: Optional[np.ndarray],
               ends: np.ndarray, seed: int, cfg: int = 0,
               dup_frac: float = 0.0, outlier_frac: float = 0.0,
               rows_to_fill=None) -> Case:
    """Allocate and fill a buffer for explicit starts/ends.

    ``rows_to_fill`` (iterable of rows) limits generation to those rows; the
    others keep the tail sentinel everywhere (useful for oracle spot checks).
    """
    buf = _alloc(shape)
    if rows_to_fill is not None:
        buf.view(np.uint32)[:] = SENTINEL_TAIL
    case = Case(name, shape, buf, starts, np.asarray(ends, dtype=np.int32), seed)
    rows = range(shape.rows) if rows_to_fill is None else rows_to_fill
    for r in rows:
        s = 0 if starts is None else int(starts[r // shape.starts_repeat])
        e = int(case.ends[r // shape.ends_repeat])
        _fill_row(buf[r], shape.col_stride, shape.width, s, e,
                  _row_rng(seed, cfg, r), shape.block_size, dup_frac, outlier_frac)
    return case


def row_values(case: Case, row: int, cfg: int, dup_frac: float = 0.0,
               outlier_frac: float = 0.0) -> np.ndarray:
    """Regenerate one row of a case (same bits as ``build_case``) by itself."""
    sh = case.shape
    tmp = np.empty(sh.width * sh.col_stride, dtype=np.float32)
    s = 0 if case.starts is None else int(case.starts[row // sh.starts_repeat])
    e = int(case.ends[row // sh.ends_repeat])
    _fill_row(tmp, sh.col_stride, sh.width, s, e, _row_rng(case.seed, cfg, row),
              sh.block_size, dup_frac, outlier_frac)
    return tmp


# --------------------------------------------------------------------------
# The five named workloads.
# --------------------------------------------------------------------------

CONFIG_SHAPES = {
    "tiny": Shape(rows=4, width=4096, block_size=8, k_blocks=64, k_tokens=256),
    "short_decode": Shape(rows=96, width=1048576, block_size=8, k_blocks=256,
                          k_tokens=2048),
    "mtp_ragged": Shape(rows=208, width=131072, block_size=16, k_blocks=128,
                        k_tokens=2048, col_stride=2, starts_repeat=4,
                        ends_repeat=1),
    "long_decode": Shape(rows=32, width=1048576, block_size=8, k_blocks=2048,
                         k_tokens=2048),
    "prefill_chunk": Shape(rows=8192, width=131072, block_size=8, k_blocks=256,
                           k_tokens=2048),
}

CONFIG_EXTRAS = {
    "tiny": dict(dup_frac=0.05),
    "short_decode": dict(),
    "mtp_ragged": dict(),
    "long_decode": dict(outlier_frac=0.01),
    "prefill_chunk": dict(),
}


def config_bounds(name: str, seed_offset: int = 0):
    """(shape, starts or None, ends, seed) for a named workload."""
    cfg = CONFIG_IDS[name]
    seed = BASE_SEED + cfg + seed_offset
    rng = np.random.default_rng([seed, cfg, 1 << 20])
    sh = CONFIG_SHAPES[name]
    W = sh.width
    if name == "tiny":
        ends = rng.integers(1, W, size=sh.rows, endpoint=True)
        ends[0], ends[1] = 1, W
        return sh, None, ends.astype(np.int32), seed
    if name == "short_decode":
        z = rng.standard_normal(sh.rows)
        ends = np.clip(np.rint(np.exp(math.log(400.0) + 0.8 * z)), 1, 8192)
        return sh, None, ends.astype(np.int32), seed
    if name == "mtp_ragged":
        nreq = sh.rows // sh.starts_repeat
        starts = rng.integers(0, 1024, size=nreq, endpoint=True)
        span = rng.integers(1, 65536, size=nreq, endpoint=True)
        base = starts + span
        starts[:4] = 0
        base[:4] = [1023, 1024, 1025, W]
        ends = np.repeat(base, sh.starts_repeat) + np.tile(
            np.arange(sh.starts_repeat), nreq)
        return sh, starts.astype(np.int32), ends.astype(np.int32), seed
    if name == "long_decode":
        ends = rng.integers(262144, W, size=sh.rows, endpoint=True)
        return sh, None, ends.astype(np.int32), seed
    if name == "prefill_chunk":
        nseq, q = 4, sh.rows // 4
        ctx = rng.integers(0, 120000, size=nseq, endpoint=True)
        ends = (ctx[:, None] + np.arange(q)[None, :] + 1).reshape(-1)
        return sh, None, np.minimum(ends, np.iinfo(np.int32).max).astype(np.int32), seed
    raise KeyError(name)


def make_config(name: str, seed_offset: int = 0, rows_to_fill=None,
                width: Optional[int] = None) -> Case:
    """A named workload; ``width`` overrides the buffer width and keeps the
    bounds and live values (each row's values depend only on the seed, the
    row and its live range)."""
    sh, starts, ends, seed = config_bounds(name, seed_offset)
    if width is not None:
        sh = dataclasses.replace(sh, width=int(width))
    return build_case(name, sh, starts, ends, seed, cfg=CONFIG_IDS[name],
                      rows_to_fill=rows_to_fill, **CONFIG_EXTRAS[name])


def make_custom(rows: int, width: int, block_size: int, k_blocks: int,
                k_tokens: int, ends, starts=None, col_stride: int = 1,
                starts_repeat: int = 1, ends_repeat: int = 1, seed: int = 1,
                dup_frac: float = 0.0, outlier_frac: float = 0.0) -> Case:
    sh = Shape(rows, width, block_size, k_blocks, k_tokens, col_stride,
               starts_repeat, ends_repeat)
    st = None if starts is None else np.asarray(starts, dtype=np.int32)
    return build_case("custom", sh, st, np.asarray(ends, dtype=np.int32), seed,
                      cfg=0, dup_frac=dup_frac, outlier_frac=outlier_frac)


# --------------------------------------------------------------------------
# Inputs of the fused indexer-logits producer (FP8 query/key codes).
# --------------------------------------------------------------------------

@dataclasses.dataclass
class IndexerCase:
    """q8 uint8 [Q, H, D] and k8 uint8 [S, D] hold OCP E4M3 codes; w float32
    [Q, H]; kscale float32 [S] or None; row t reads starts[t // starts_repeat]
    (None: 0) and ends[t // ends_repeat]."""
    name: str
    q8: np.ndarray
    k8: np.ndarray
    w: np.ndarray
    kscale: Optional[np.ndarray]
    starts: Optional[np.ndarray]
    ends: np.ndarray
    block_size: int
    k_blocks: int
    k_tokens: int
    starts_repeat: int = 1
    ends_repeat: int = 1

    @property
    def queries(self) -> int:
        return self.q8.shape[0]

    @property
    def heads(self) -> int:
        return self.q8.shape[1]

    @property
    def head_dim(self) -> int:
        return self.q8.shape[2]

    @property
    def keys(self) -> int:
        return self.k8.shape[0]


def e4m3_codes(rng: np.random.Generator, shape, exp_lo: int = 5, exp_hi: int = 7) -> np.ndarray:
    """Random E4M3 bytes: random sign, exponent field in [exp_lo, exp_hi],
    random 3-bit mantissa (bit fields only; no value arithmetic)."""
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8) << 7
    expo = rng.integers(exp_lo, exp_hi + 1, size=shape, dtype=np.uint8) << 3
    mant = rng.integers(0, 8, size=shape, dtype=np.uint8)
    return (sign | expo | mant).astype(np.uint8)


def make_indexer_custom(queries: int, keys: int, heads: int, head_dim: int, block_size: int,
                        k_blocks: int, k_tokens: int, ends, starts=None, seed: int = 1,
                        with_kscale: bool = True, starts_repeat: int = 1,
                        ends_repeat: int = 1, name: str = "indexer_custom") -> IndexerCase:
    """Seeded synthetic indexer inputs.  Query and key codes have exponent
    fields 5..7 (magnitudes 0.25..1.875), head weights are +-n/16 with n in
    1..16, and key scales are 1, 1/2 or 1/4."""
    rng = np.random.default_rng([seed, 48726])
    q8 = e4m3_codes(rng, (queries, heads, head_dim))
    k8 = e4m3_codes(rng, (keys, head_dim))
    n = rng.integers(1, 17, size=(queries, heads)).astype(np.float32)
    sgn = np.where(rng.integers(0, 2, size=(queries, heads)) == 1, 1.0, -1.0).astype(np.float32)
    w = (sgn * n / np.float32(16.0)).astype(np.float32)
    kscale = None
    if with_kscale:
        kscale = np.ldexp(np.ones(keys, np.float32),
                          -rng.integers(0, 3, size=keys)).astype(np.float32)
    st = None if starts is None else np.asarray(starts, dtype=np.int32)
    return IndexerCase(name, q8, k8, w, kscale, st, np.asarray(ends, dtype=np.int32),
                       block_size, k_blocks, k_tokens, starts_repeat, ends_repeat)


INDEXER_CONFIGS = {
    # a prefill chunk of 8192 queries at the end of a 262,144-token context,
    # 64 indexer heads of dimension 128, top-256 blocks of 8 then top-2048 tokens
    "indexer_prefill": dict(queries=8192, keys=262144, heads=64, head_dim=128,
                            block_size=8, k_blocks=256, k_tokens=2048),
    # the same per-row work on a chunk of 256 queries (parity-sized)
    "indexer_small": dict(queries=256, keys=65536, heads=64, head_dim=128,
                          block_size=8, k_blocks=256, k_tokens=2048),
}


def make_indexer_config(name: str, seed_offset: int = 0) -> IndexerCase:
    """Causal bounds: query t of a chunk of Q at the end of S keys sees keys
    [0, S - Q + t + 1)."""
    c = INDEXER_CONFIGS[name]
    Q, S = c["queries"], c["keys"]
    ends = (S - Q + np.arange(Q) + 1).astype(np.int32)
    return make_indexer_custom(Q, S, c["heads"], c["head_dim"], c["block_size"],
                               c["k_blocks"], c["k_tokens"], ends,
                               seed=BASE_SEED + 100 + seed_offset, name=name)


# --------------------------------------------------------------------------
# Inputs of the sparse attention over each row's selected tokens.
# --------------------------------------------------------------------------

def bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 codes (round to nearest even on the bit
    pattern; the inputs here are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@dataclasses.dataclass
class AttnCase:
    """q uint16 bf16 [R, Hkv * G, D]; k_cache / v_cache uint16 bf16
    [num_slots, Hkv, D] (None when the caches are generated on the device
    from ``cache_seed``); token_ids int32 [R, K] ascending with -1 pads;
    page_table int32 [num_seqs, pages_per_seq] (-1: unmapped) or None; row r
    belongs to sequence r // rows_per_seq; gate uint16 bf16 like q, or None."""
    name: str
    q: np.ndarray
    k_cache: Optional[np.ndarray]
    v_cache: Optional[np.ndarray]
    token_ids: np.ndarray
    page_table: Optional[np.ndarray]
    page_size: int
    rows_per_seq: int
    gate: Optional[np.ndarray]
    kv_heads: int
    group: int
    head_dim: int
    sm_scale: float
    num_slots: int
    seq_lens: np.ndarray
    cache_seed: int = 0
    k_scale: Optional[float] = None   # fp8 caches: uint8 E4M3 codes times these scales
    v_scale: Optional[float] = None

    @property
    def kv_fp8(self) -> bool:
        return self.k_scale is not None

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def k_tokens(self) -> int:
        return self.token_ids.shape[1]


def _sorted_sample(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """k distinct integers of [0, n), ascending."""
    if k >= n:
        return np.arange(n, dtype=np.int64)
    if n <= 4 * k:
        return np.sort(rng.permutation(n)[:k])
    picked = np.unique(rng.integers(0, n, size=k + k // 4 + 16))
    while picked.size < k:
        picked = np.unique(np.concatenate([picked, rng.integers(0, n, size=k)]))
    return np.sort(rng.permutation(picked)[:k])


def make_attn_custom(seq_lens, rows_per_seq: int, kv_heads: int, group: int, head_dim: int,
                     k_tokens: int, page_size: int = 16, paged: bool = True,
                     with_gate: bool = True, seed: int = 1, q_scale: float = 1.0,
                     host_caches: bool = True, spare_pages: int = 3, kv_fp8: bool = False,
                     shared: float = 0.0, name: str = "attn_custom") -> AttnCase:
    """Seeded synthetic attention inputs.

    Sequence n has seq_lens[n] cached positions; its rows_per_seq rows are
    consecutive query tokens (multi-token prediction), row j seeing the first
    seq_lens[n] - (rows_per_seq - 1 - j) positions.  Each row selects
    min(k_tokens, visible) distinct positions uniformly, ascending, padded
    with -1.  Pages are scattered: a random permutation of the physical pages
    (plus ``spare_pages`` never mapped) backs the sequences, and table
    entries past a sequence's length are -1.  q, K, V and the gate are
    N(0, 1) rounded to bf16 (q times ``q_scale``); the softmax scale is
    1 / sqrt(head_dim).  With ``kv_fp8`` the caches hold E4M3 codes (random
    sign, exponent field 3..9, random mantissa: magnitudes 1/16..7.5) with
    k_scale 1/4 and v_scale 1/2.  With ``shared`` > 0 the rows of a request
    select overlapping sets, as neighbouring queries do: the request draws a
    base set of min(k_tokens, visible) positions that all its rows see, and
    each row keeps round(shared * k) of them (a random subset) and draws the
    rest uniformly from its other visible positions.
    """
    rng = np.random.default_rng([seed, 57273])
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    nseq = seq_lens.size
    R = nseq * rows_per_seq
    hq = kv_heads * group
    pages = [int(-(-int(L) // page_size)) for L in seq_lens]
    if paged:
        total = sum(pages) + spare_pages
        perm = rng.permutation(total).astype(np.int32)
        pps = max(1, max(pages) if pages else 1)
        table = np.full((nseq, pps), -1, dtype=np.int32)
        at = 0
        for n, p in enumerate(pages):
            table[n, :p] = perm[at:at + p]
            at += p
        num_slots = total * page_size
    else:
        table = None
        num_slots = int(seq_lens.max()) if nseq else 0
    ids = np.full((R, k_tokens), -1, dtype=np.int32)
    for n in range(nseq):
        vis0 = max(0, int(seq_lens[n]) - (rows_per_seq - 1))
        base = _sorted_sample(rng, vis0, min(k_tokens, vis0)) if shared > 0 else None
        for j in range(rows_per_seq):
            vis = max(0, int(seq_lens[n]) - (rows_per_seq - 1 - j))
            k = min(k_tokens, vis)
            if base is not None and base.size:
                keep = min(int(round(shared * k)), base.size)
                kept = rng.choice(base, size=keep, replace=False)
                pool = np.setdiff1d(np.arange(vis), kept)
                extra = pool[_sorted_sample(rng, pool.size, k - keep)]
                pick = np.sort(np.concatenate([kept, extra]))
            else:
                pick = _sorted_sample(rng, vis, k)
            ids[n * rows_per_seq + j, :pick.size] = pick
    q = bf16_bits(rng.standard_normal((R, hq, head_dim), dtype=np.float32) * np.float32(q_scale))
    gate = bf16_bits(rng.standard_normal((R, hq, head_dim), dtype=np.float32)) if with_gate else None
    kc = vc = None
    if host_caches:
        shape = (num_slots, kv_heads, head_dim)
        if kv_fp8:
            kc = e4m3_codes(rng, shape, 3, 9)
            vc = e4m3_codes(rng, shape, 3, 9)
        else:
            kc = bf16_bits(rng.standard_normal(shape, dtype=np.float32))
            vc = bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    return AttnCase(name, q, kc, vc, ids, table, page_size, rows_per_seq, gate, kv_heads, group,
                    head_dim, 1.0 / math.sqrt(head_dim), num_slots, seq_lens,
                    cache_seed=seed, k_scale=0.25 if kv_fp8 else None,
                    v_scale=0.5 if kv_fp8 else None)


ATTN_CONFIGS = {
    # decode at 128 concurrent requests with 3 draft tokens (4 query rows per
    # request), 2 kv heads of 256 dimensions with 12 query heads each, the
    # 2048 selected tokens of each row out of contexts of 32K-128K tokens
    # (5% of requests shorter than 2048), a 64-token paged cache and an
    # output gate; the K/V caches (about 21 GB) are generated on the device
    "attn_decode": dict(num_seqs=128, rows_per_seq=4, kv_heads=2, group=12, head_dim=256,
                        k_tokens=2048, page_size=64, ctx=(32768, 131072), short_frac=0.05,
                        host_caches=False),
    # the same decode batch over fp8 (E4M3) K/V caches with per-tensor scales
    "attn_decode_fp8": dict(num_seqs=128, rows_per_seq=4, kv_heads=2, group=12, head_dim=256,
                            k_tokens=2048, page_size=64, ctx=(32768, 131072), short_frac=0.05,
                            host_caches=False, kv_fp8=True),
    # one request (4 rows), 1 kv head with 3 query heads: the latency case
    "attn_c1": dict(num_seqs=1, rows_per_seq=4, kv_heads=1, group=3, head_dim=256,
                    k_tokens=2048, page_size=64, ctx=(65536, 65536), short_frac=0.0,
                    host_caches=False),
    # the decode point of the QSA tuning page's benchmark (128 requests, 4
    # query rows each, 3 query heads per kv head, 1 kv head), with the rows
    # of a request sharing 3/4 of their selections (neighbouring queries
    # select overlapping positions); the union form packs a request's 4 x 3
    # (row, head) pairs into one matrix tile
    "attn_decode_g3": dict(num_seqs=128, rows_per_seq=4, kv_heads=1, group=3, head_dim=256,
                           k_tokens=2048, page_size=64, ctx=(32768, 131072), short_frac=0.05,
                           host_caches=False, shared=0.75),
    # parity-sized form of it: 8 requests, host caches
    "attn_small_g3": dict(num_seqs=8, rows_per_seq=4, kv_heads=1, group=3, head_dim=256,
                          k_tokens=2048, page_size=64, ctx=(1, 12000), short_frac=0.25,
                          host_caches=True, q_scale=3.0, shared=0.75),
    # parity-sized: 8 requests x 4 rows, host caches, queries scaled by 3 so
    # that each softmax concentrates on a few tokens
    "attn_small": dict(num_seqs=8, rows_per_seq=4, kv_heads=2, group=12, head_dim=256,
                       k_tokens=2048, page_size=64, ctx=(1, 12000), short_frac=0.25,
                       host_caches=True, q_scale=3.0),
}


def make_attn_config(name: str, seed_offset: int = 0) -> AttnCase:
    c = ATTN_CONFIGS[name]
    rng = np.random.default_rng([BASE_SEED + 200 + seed_offset, len(name)])
    lo, hi = c["ctx"]
    lens = rng.integers(lo, hi + 1, size=c["num_seqs"])
    short = rng.random(c["num_seqs"]) < c["short_frac"]
    lens = np.where(short, rng.integers(1, c["k_tokens"] + 1, size=c["num_seqs"]), lens)
    return make_attn_custom(lens, c["rows_per_seq"], c["kv_heads"], c["group"], c["head_dim"],
                            c["k_tokens"], page_size=c["page_size"],
                            seed=BASE_SEED + 200 + seed_offset, host_caches=c["host_caches"],
                            q_scale=c.get("q_scale", 1.0), kv_fp8=c.get("kv_fp8", False),
                            shared=c.get("shared", 0.0), name=name)
