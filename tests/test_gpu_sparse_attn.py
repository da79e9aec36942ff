"""Parity of the sparse attention over each row's selected tokens (needs an MI355X).

The kernel's bf16 outputs and fp32 log-sum-exps are compared with the oracle
(float64, tests/test_sparse_attn_oracle.py pins it) element by element, within
a bound derived from the kernel's arithmetic:

* The softmax weights p_j are rounded to bf16 (relative error <= 2^-8) before
  they multiply V, and the output is rounded to bf16 (relative <= 2^-8).  The
  scores are fp32 sums of exact bf16 products (over 256 dimensions the sum's
  error stays below 2^-16 of sum |q_i k_i|, a few 1e-4 for these inputs),
  which moves each weight by a relative 2^-11 or so.  Hence per element
      |out - ref| <= 2^-7 * A + 2^-8 * |ref|,
  A = sum_j p_j |v_j| * sigmoid(gate) (the oracle's attention over |V|), which
  covers the first-order terms 2^-8 A + 2^-10 A with room to spare.
* lse: |lse - ref| <= 2^-16 * sm_scale * max_j sum_i |q_i k_ji| + 2^-11
  (score sums, the fp32 sum of up to 2048 weights and the hardware log2).
Rows without a token give exactly 0 and -inf.  The page's own check is
rtol = atol = 2e-2 against an fp32 reference; this bound is tighter.
"""
import math

import numpy as np
import pytest

from oracle import sparse_attn_oracle as so
from sparse_attention_indexer_start_amd import binding
from sparse_attention_indexer_start_amd import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load()
    yield
    torch.cuda.synchronize()


def _bf(a):
    """uint16 bf16 codes (numpy) -> bf16 device tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _codes(t):
    return t.view(__import__("torch").int16).cpu().numpy().view(np.uint16)


def _f(codes):
    return (codes.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _cache_dev(a):
    """A host cache (bf16 codes or E4M3 bytes) on the device."""
    import torch
    if a.dtype == np.uint8:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return _bf(a)


def _run(case, k_dev=None, v_dev=None, chunks=0, with_gate=True, with_lse=True, union_rows=0):
    import torch
    hq = case.kv_heads * case.group
    kd = _cache_dev(case.k_cache) if k_dev is None else k_dev
    vd = _cache_dev(case.v_cache) if v_dev is None else v_dev
    pps = 0 if case.page_table is None else case.page_table.shape[1]
    op = binding.SparseAttn(case.rows, case.kv_heads, case.group, case.head_dim, case.k_tokens,
                            case.num_slots, rows_per_seq=case.rows_per_seq,
                            page_size=case.page_size, pages_per_seq=pps,
                            k_strides=(kd.stride(0), kd.stride(1)),
                            v_strides=(vd.stride(0), vd.stride(1)), chunks=chunks,
                            union_rows=union_rows)
    q = _bf(case.q)
    gate = _bf(case.gate) if (with_gate and case.gate is not None) else None
    ids = torch.from_numpy(case.token_ids).cuda()
    table = None if case.page_table is None else torch.from_numpy(case.page_table).cuda()
    out = torch.empty((case.rows, hq, case.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((case.rows, hq), float("nan"), device="cuda") if with_lse else None
    op(q, kd, vd, ids, table, gate, case.sm_scale, out, lse, k_scale=case.k_scale,
       v_scale=case.v_scale)
    torch.cuda.synchronize()
    status = op.read_status()
    gh.log(f"  attention: {case.rows} rows, {case.kv_heads}x{case.group} heads, D={case.head_dim}, "
           f"K={case.k_tokens}, {'fp8' if case.kv_fp8 else 'bf16'} K/V, {op.chunks()} chunks, "
           f"union_rows {union_rows}, status {status}")
    op.close()
    return _codes(out), (None if lse is None else lse.cpu().numpy()), status


def _check(case, got_codes, got_lse, rows=None, with_gate=True, distinct=False):
    gate = case.gate if with_gate else None
    args = (case.q, case.k_cache, case.v_cache, case.token_ids, case.sm_scale, case.group,
            case.page_table, case.page_size, case.rows_per_seq)
    sc = dict(k_scale=case.k_scale, v_scale=case.v_scale, distinct=distinct)
    ref, ref_lse, bad = so.sparse_attention(*args, gate=gate, rows=rows, **sc)
    sign_off = np.uint8(0x7F) if case.kv_fp8 else np.uint16(0x7FFF)
    A, _, _ = so.sparse_attention(case.q, case.k_cache, case.v_cache & sign_off, *args[3:],
                                  gate=gate, rows=rows, **sc)
    got = _f(got_codes)
    rows = range(case.rows) if rows is None else rows
    if case.kv_fp8:
        from oracle import indexer_oracle
        kd = indexer_oracle.e4m3_decode(case.k_cache) * case.k_scale
    else:
        kd = so.bf16_decode(case.k_cache)
    for r in rows:
        tol = 2.0 ** -7 * A[r] + 2.0 ** -8 * np.abs(ref[r])
        err = np.abs(got[r] - ref[r])
        assert np.all(err <= tol), (f"row {r}: worst excess {np.max(err - tol):.3e} at "
                                    f"{np.unravel_index(np.argmax(err - tol), err.shape)}")
        if got_lse is None:
            continue
        if np.all(np.isinf(ref_lse[r])):
            assert np.all(got_lse[r] == -np.inf) and np.all(got[r] == 0.0), f"row {r}: empty row"
            continue
        seq = r // case.rows_per_seq
        slots = [so.slot_of(p, seq, case.page_table, case.page_size, case.num_slots)
                 for p in case.token_ids[r] if p >= 0]
        slots = np.array([s for s in slots if s >= 0])
        qd = np.abs(so.bf16_decode(case.q[r]))
        for h in range(case.kv_heads * case.group):
            g = h // case.group
            mx = (np.abs(kd[slots, g, :]) @ qd[h]).max()
            tl = 2.0 ** -16 * case.sm_scale * mx + 2.0 ** -11
            assert abs(got_lse[r, h] - ref_lse[r, h]) <= tl, (r, h, got_lse[r, h], ref_lse[r, h])
    return bad


def test_attn_small_config_every_row():
    case = wl.make_attn_config("attn_small")
    got, lse, status = _run(case)
    assert status == 0
    _check(case, got, lse)


@pytest.mark.parametrize("D,G,hkv,K,chunks,paged,gate,with_lse", [
    (256, 1, 1, 33, 0, True, False, True),
    (256, 3, 1, 2048, 1, True, True, True),
    (256, 16, 2, 300, 3, False, True, True),
    (128, 6, 2, 1000, 0, True, True, False),
    (128, 16, 1, 64, 2, True, False, True),
    (256, 12, 2, 2048, 64, True, True, True),
    (128, 5, 3, 1, 0, True, True, True),
    (128, 2, 4, 700, 0, True, True, True),
    (256, 4, 6, 200, 2, True, True, True),
    (256, 8, 8, 2048, 0, True, False, True),
    # groups above one matrix tile: 2, 8, 3 and 5 head tiles per kv head
    (128, 32, 1, 500, 0, True, True, True),
    (128, 128, 1, 300, 0, True, True, True),
    (256, 24, 2, 700, 3, True, True, True),
    (128, 17, 2, 200, 0, True, False, True),
])
def test_attn_shapes(D, G, hkv, K, chunks, paged, gate, with_lse):
    rng = np.random.default_rng(D + 7 * G + 11 * K)
    lens = rng.integers(1, 3 * K + 40, size=3)
    lens[0] = 1
    case = wl.make_attn_custom(lens, 3, hkv, G, D, K, page_size=16, paged=paged,
                               with_gate=gate, seed=G * 100 + K, q_scale=2.0)
    got, lse, status = _run(case, chunks=chunks, with_gate=gate, with_lse=with_lse)
    assert status == 0
    _check(case, got, lse, with_gate=gate)


def test_attn_strided_caches():
    """Caches as views with padded heads and slots (strides in elements)."""
    import torch
    case = wl.make_attn_custom([700, 1500], 2, 2, 8, 256, 512, page_size=32, seed=21,
                               q_scale=2.0)
    big_k = torch.zeros((case.num_slots, 3, 256 + 64), dtype=torch.bfloat16, device="cuda")
    big_v = torch.zeros((case.num_slots, 2, 256 + 128), dtype=torch.bfloat16, device="cuda")
    kv = big_k[:, :2, :256]
    vv = big_v[:, :, 64:320]
    kv.copy_(_bf(case.k_cache))
    vv.copy_(_bf(case.v_cache))
    got, lse, status = _run(case, k_dev=kv, v_dev=vv)
    assert status == 0
    _check(case, got, lse)


def test_attn_empty_rows_and_unaddressable_ids():
    case = wl.make_attn_custom([5, 300, 2], 2, 1, 4, 256, 64, page_size=16, seed=23)
    case.token_ids[0, :] = -1                        # no token at all
    case.token_ids[3, 5] = 10_000                    # page beyond the table
    case.token_ids[5, 2] = 20                        # page 1 of a 2-position sequence: unmapped
    got, lse, status = _run(case, chunks=2)
    assert status & 1, "unaddressable ids must set status bit 0"
    bad = _check(case, got, lse)
    assert bad[3] == 1 and bad[5] == 1 and bad.sum() == 2
    assert np.all(_f(got[0]) == 0.0) and np.all(lse[0] == -np.inf)


def test_attn_graph_replay_with_new_ids():
    import torch
    case = wl.make_attn_custom([3000, 2500, 4000, 100], 2, 2, 6, 256, 1024, page_size=64,
                               seed=25, q_scale=2.0)
    hq = case.kv_heads * case.group
    op = binding.SparseAttn(case.rows, case.kv_heads, case.group, 256, case.k_tokens,
                            case.num_slots, rows_per_seq=2, page_size=64,
                            pages_per_seq=case.page_table.shape[1])
    q, kd, vd, gate = _bf(case.q), _bf(case.k_cache), _bf(case.v_cache), _bf(case.gate)
    ids = torch.from_numpy(case.token_ids).cuda()
    table = torch.from_numpy(case.page_table).cuda()
    out = torch.empty((case.rows, hq, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((case.rows, hq), device="cuda")
    op(q, kd, vd, ids, table, gate, case.sm_scale, out, lse)
    torch.cuda.synchronize()
    first = _codes(out).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op(q, kd, vd, ids, table, gate, case.sm_scale, out, lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(25)
    for it in range(6):
        if it % 2 == 0:
            new = case.token_ids.copy()
        else:
            other = wl.make_attn_custom(case.seq_lens, 2, 2, 6, 256, 1024, page_size=64,
                                        seed=100 + it, host_caches=False)
            new = other.token_ids
        ids.copy_(torch.from_numpy(new))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if it % 2 == 0:
            assert np.array_equal(_codes(out), first), f"replay {it} differs from the eager call"
        else:
            c2 = wl.AttnCase(**{**case.__dict__, "token_ids": new})
            _check(c2, _codes(out), lse.cpu().numpy())
    assert op.read_status() == 0
    op.close()


def _device_caches(case):
    import bench
    return bench.attn_device_caches(case)


def _gathered_case(case, kd, vd, rows):
    """The given rows with their attended slots copied from the device caches
    into a compact host cache (ids renumbered, no page table)."""
    import torch
    slots, ids = [], np.full((len(rows), case.k_tokens), -1, np.int32)
    for i, r in enumerate(rows):
        seq = r // case.rows_per_seq
        s = [so.slot_of(p, seq, case.page_table, case.page_size, case.num_slots)
             for p in case.token_ids[r] if p >= 0]
        assert all(x >= 0 for x in s)
        ids[i, :len(s)] = np.arange(len(slots), len(slots) + len(s))
        slots.extend(s)
    idx = torch.tensor(slots if slots else [0], dtype=torch.int64, device="cuda")
    if case.kv_fp8:
        kc = kd.index_select(0, idx).cpu().numpy()
        vc = vd.index_select(0, idx).cpu().numpy()
    else:
        kc = _codes(kd.index_select(0, idx))
        vc = _codes(vd.index_select(0, idx))
    rows = list(rows)
    return wl.AttnCase("gathered", case.q[rows], kc, vc, ids, None, 1, 1,
                       None if case.gate is None else case.gate[rows], case.kv_heads,
                       case.group, case.head_dim, case.sm_scale, max(1, len(slots)),
                       case.seq_lens, k_scale=case.k_scale, v_scale=case.v_scale)


@pytest.mark.parametrize("name", ["attn_decode", "attn_c1", "attn_decode_fp8"])
def test_attn_full_size_sampled_rows(name):
    import torch
    case = wl.make_attn_config(name)
    gh.log(f"{name}: {case.rows} rows, {case.num_slots} slots")
    kd, vd = _device_caches(case)
    got, lse, status = _run(case, k_dev=kd, v_dev=vd)
    assert status == 0
    valid = (case.token_ids >= 0).sum(1)
    rng = np.random.default_rng(3)
    rows = sorted(set([0, case.rows - 1] + list(np.nonzero(valid < case.k_tokens)[0][:8])
                      + list(rng.choice(case.rows, size=min(case.rows, 24), replace=False))))
    gc = _gathered_case(case, kd, vd, rows)
    _check(gc, got[rows], lse[rows])
    # every row: finite output, lse finite exactly where the row has tokens
    allf = _f(got)
    assert np.all(np.isfinite(allf))
    assert np.array_equal(np.isfinite(lse).all(1), valid > 0)
    del kd, vd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("D,G,hkv,K,chunks", [
    (256, 12, 2, 2048, 0), (256, 3, 1, 300, 4), (128, 16, 2, 700, 0), (128, 5, 3, 33, 1),
    (128, 64, 1, 500, 0),
])
def test_attn_fp8_caches(D, G, hkv, K, chunks):
    rng = np.random.default_rng(D + G + K)
    lens = rng.integers(1, 3 * K + 40, size=3)
    case = wl.make_attn_custom(lens, 2, hkv, G, D, K, page_size=32, seed=G + K, q_scale=0.5,
                               kv_fp8=True)
    got, lse, status = _run(case, chunks=chunks)
    assert status == 0
    _check(case, got, lse)


def test_attn_rejects_unsupported_shapes():
    with pytest.raises(binding.DsaError):
        binding.SparseAttn(4, 1, 0, 256, 64, 100)            # group 0
    with pytest.raises(binding.DsaError):
        binding.SparseAttn(4, 1, 4, 64, 64, 100)            # head_dim 64
    with pytest.raises(binding.DsaError):
        binding.SparseAttn(4, 1, 4, 256, 64, 100, page_size=3)
    with pytest.raises(binding.DsaError):
        binding.SparseAttn(4, 2, 4, 256, 64, 100, k_strides=(516, 256))   # not a multiple of 8


# ---------------------------------------------------------------------------
# Union mode: groups of rows over the union of their ids, each row exact
# ---------------------------------------------------------------------------

def test_attn_union_small_config_every_row():
    case = wl.make_attn_config("attn_small_g3")
    got, lse, status = _run(case, union_rows=4)
    assert status == 0
    _check(case, got, lse, distinct=True)
    # the per-row form of the same inputs agrees with the same oracle
    got1, lse1, status1 = _run(case)
    assert status1 == 0
    _check(case, got1, lse1)


@pytest.mark.parametrize("D,G,hkv,K,U,rps,chunks,paged,gate,shared", [
    (256, 3, 1, 2048, 4, 4, 0, True, True, 0.75),
    (256, 3, 1, 300, 5, 5, 3, True, True, 0.5),
    (128, 8, 2, 700, 2, 4, 0, False, True, 0.9),
    (128, 1, 4, 100, 16, 16, 0, True, False, 0.75),
    (256, 6, 3, 1000, 2, 2, 1, True, True, 0.75),
    (128, 2, 1, 2048, 8, 8, 64, True, True, 0.6),
    (256, 4, 2, 4096, 4, 8, 0, True, True, 0.75),
    (128, 1, 1, 2048, 16, 16, 0, True, True, 0.0),
    # union_rows * group above 16: the group's heads in 4, 5, 3 and 2 tiles
    (128, 16, 1, 500, 4, 4, 0, True, True, 0.75),
    (256, 5, 1, 300, 4, 4, 2, True, True, 0.5),
    (256, 12, 2, 400, 4, 8, 0, True, True, 0.75),
    (128, 6, 1, 1000, 4, 4, 0, True, False, 0.75),
])
def test_attn_union_shapes(D, G, hkv, K, U, rps, chunks, paged, gate, shared):
    rng = np.random.default_rng(D + 7 * G + 11 * K + U)
    lens = rng.integers(1, 3 * K + 40, size=3)
    lens[0] = 1
    case = wl.make_attn_custom(lens, rps, hkv, G, D, K, page_size=16, paged=paged,
                               with_gate=gate, seed=G * 100 + K + U, q_scale=2.0, shared=shared)
    got, lse, status = _run(case, chunks=chunks, with_gate=gate, union_rows=U)
    assert status == 0
    _check(case, got, lse, with_gate=gate, distinct=True)


def test_attn_union_many_windows():
    """Positions spread over several of the union kernel's 262144-position
    windows (contexts of 270K-600K tokens), with windows left empty."""
    case = wl.make_attn_custom([600000, 300000, 270000, 5], 4, 1, 3, 128, 1024, page_size=64,
                               seed=31, q_scale=2.0, shared=0.5)
    ids = case.token_ids
    ids[4:8] = np.where(ids[4:8] >= 262144, ids[4:8], -1)    # request 1: its second window only
    got, lse, status = _run(case, chunks=2, union_rows=4)
    assert status == 0
    _check(case, got, lse, distinct=True)


def test_attn_union_repeats_pads_order_and_bad_ids():
    """Ids in any order, repeated within a row (counted once), -1 pads
    anywhere, a whole group without ids, a short last group, and ids that
    are not addressable (skipped, status bit 0)."""
    case = wl.make_attn_custom([900, 3, 2500, 40], 4, 2, 3, 256, 512, page_size=16, seed=27,
                               q_scale=2.0, shared=0.5)
    rng = np.random.default_rng(27)
    ids = case.token_ids
    for r in range(ids.shape[0]):
        rng.shuffle(ids[r])                              # any order, pads scattered
    ids[0, :40] = ids[0, 100]                            # one id forty times
    ids[2, 7] = ids[2, 9] if ids[2, 9] >= 0 else ids[2, 7]
    ids[4:8, :] = -1                                     # group 1 holds no id
    ids[9, 3] = 10_000                                   # page beyond the table
    ids[13, 0] = 50                                      # page 3 of a 40-token sequence: unmapped
    keep = ids.shape[0] - 1                              # the last group has 3 rows
    c2 = wl.AttnCase(**{**case.__dict__, "q": case.q[:keep], "token_ids": ids[:keep].copy(),
                        "gate": case.gate[:keep]})
    got, lse, status = _run(c2, chunks=3, union_rows=4)
    assert status & 1, "unaddressable ids must set status bit 0"
    bad = _check(c2, got, lse, distinct=True)
    assert bad[9] == 1 and bad[13] == 1 and bad.sum() == 2
    assert np.all(_f(got[4:8]) == 0.0) and np.all(lse[4:8] == -np.inf)


@pytest.mark.parametrize("D,G,hkv,K,U,chunks", [(256, 3, 1, 1000, 4, 0), (128, 4, 2, 300, 4, 2)])
def test_attn_union_fp8_caches(D, G, hkv, K, U, chunks):
    rng = np.random.default_rng(D + G + K + 1)
    lens = rng.integers(1, 3 * K + 40, size=3)
    case = wl.make_attn_custom(lens, 4, hkv, G, D, K, page_size=32, seed=G + K + 1,
                               q_scale=0.5, kv_fp8=True, shared=0.75)
    got, lse, status = _run(case, chunks=chunks, union_rows=U)
    assert status == 0
    _check(case, got, lse, distinct=True)


def test_attn_union_graph_replay_with_new_ids():
    """The two launches of union mode under graph capture: replays follow
    new ids, and a replay of the first ids repeats the eager call bit for bit."""
    import torch
    case = wl.make_attn_custom([3000, 2500, 4000, 100], 4, 1, 3, 256, 1024, page_size=64,
                               seed=29, q_scale=2.0, shared=0.75)
    hq = case.kv_heads * case.group
    op = binding.SparseAttn(case.rows, 1, 3, 256, case.k_tokens, case.num_slots, rows_per_seq=4,
                            page_size=64, pages_per_seq=case.page_table.shape[1], union_rows=4)
    q, kd, vd, gate = _bf(case.q), _bf(case.k_cache), _bf(case.v_cache), _bf(case.gate)
    ids = torch.from_numpy(case.token_ids).cuda()
    table = torch.from_numpy(case.page_table).cuda()
    out = torch.empty((case.rows, hq, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((case.rows, hq), device="cuda")
    op(q, kd, vd, ids, table, gate, case.sm_scale, out, lse)
    torch.cuda.synchronize()
    first = _codes(out).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op(q, kd, vd, ids, table, gate, case.sm_scale, out, lse)
    torch.cuda.synchronize()
    for it in range(6):
        if it % 2 == 0:
            new = case.token_ids.copy()
        else:
            other = wl.make_attn_custom(case.seq_lens, 4, 1, 3, 256, 1024, page_size=64,
                                        seed=200 + it, host_caches=False, shared=0.2 * it)
            new = other.token_ids
        ids.copy_(torch.from_numpy(new))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if it % 2 == 0:
            assert np.array_equal(_codes(out), first), f"replay {it} differs from the eager call"
        else:
            c2 = wl.AttnCase(**{**case.__dict__, "token_ids": new})
            _check(c2, _codes(out), lse.cpu().numpy(), distinct=True)
    assert op.read_status() == 0
    op.close()


def test_attn_union_full_size_sampled_rows():
    """The decode batch of 128 requests x 4 rows, 1 kv head x 3 query heads,
    in union mode over device caches; sampled rows against the oracle."""
    import torch
    case = wl.make_attn_config("attn_decode_g3")
    gh.log(f"attn_decode_g3: {case.rows} rows, {case.num_slots} slots, union of 4 rows")
    kd, vd = _device_caches(case)
    got, lse, status = _run(case, k_dev=kd, v_dev=vd, union_rows=4)
    assert status == 0
    valid = (case.token_ids >= 0).sum(1)
    rng = np.random.default_rng(5)
    rows = sorted(set([0, 1, 2, 3, case.rows - 1] + list(np.nonzero(valid < case.k_tokens)[0][:8])
                      + list(rng.choice(case.rows, size=24, replace=False))))
    gc = _gathered_case(case, kd, vd, rows)
    _check(gc, got[rows], lse[rows])
    assert np.all(np.isfinite(_f(got)))
    assert np.array_equal(np.isfinite(lse).all(1), valid > 0)
    del kd, vd
    torch.cuda.empty_cache()


def _attn_fuzz_case(seed):
    rng = np.random.default_rng(9000 + seed)
    D = int(rng.choice([128, 256]))
    hkv = int(rng.choice([1, 2, 3, 4]))
    G = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 20, 24, 32, 40]))
    U = int(rng.choice([0, 0, 2, 3, 4, 8]))
    rps = max(U, 1) * int(rng.choice([1, 2]))
    K = int(rng.integers(1, 1500))
    chunks = int(rng.choice([0, 0, 1, 2, 5]))
    lens = rng.integers(1, 3 * K + 40, size=int(rng.integers(1, 4)))
    case = wl.make_attn_custom(lens, rps, hkv, G, D, K, page_size=int(rng.choice([16, 64])),
                               paged=bool(rng.random() < 0.8), with_gate=bool(rng.random() < 0.7),
                               seed=seed, q_scale=2.0, kv_fp8=bool(rng.random() < 0.3),
                               shared=float(rng.choice([0.0, 0.5, 0.75])))
    return case, U, chunks


@pytest.mark.parametrize("seed", range(32))
def test_attn_fuzz(seed):
    """Random shapes: head_dim, kv heads, 1-40 query heads per kv head (head
    tiles), per-row or union mode with 2-8 rows per group, 1-1500 ids,
    chunk counts, paged or flat, bf16 or fp8 caches, gate on or off."""
    case, U, chunks = _attn_fuzz_case(seed)
    gate = case.gate is not None
    got, lse, status = _run(case, chunks=chunks, with_gate=gate, union_rows=U)
    assert status == 0
    _check(case, got, lse, with_gate=gate, distinct=U > 1)


def test_attn_union_rejects():
    with pytest.raises(binding.DsaError):
        binding.SparseAttn(34, 1, 1, 256, 64, 100, rows_per_seq=17, union_rows=17)  # 17 rows
    with pytest.raises(binding.DsaError):
        binding.SparseAttn(8, 1, 3, 256, 8193, 100, rows_per_seq=4, union_rows=4)  # 32772 ids
    with pytest.raises(binding.DsaError):
        binding.SparseAttn(8, 1, 3, 256, 64, 100, rows_per_seq=6, union_rows=4)    # straddles
