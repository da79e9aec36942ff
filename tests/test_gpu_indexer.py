"""Parity of the fused FP8 indexer-logits producer plus selection (needs an MI355X).

Every comparison is bit-exact: block ids, token ids and, through the
``logits_out`` testing aid, the logits themselves against the indexer oracle
(float64 evaluation rounded once to float32; the seeded inputs keep every
partial sum exact, so the kernel's fp32 sums agree bit for bit).  Rows with
empty, partial and clamped ranges, non-zero starts and repeats, all-equal
logits (every block ties), both token routes (closed form and recomputed
kept columns) and rows long enough to refill the candidate buffer many times
are covered; the parity-sized chunk is compared on every row and the
prefill-sized chunk on sampled rows.
"""
import numpy as np
import pytest

from oracle import indexer_oracle as io
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


def _to_dev(case):
    import torch
    d = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return d(case.q8), d(case.k8), d(case.w), d(case.kscale), d(case.starts), d(case.ends)


def _run(case, with_logits=True):
    import torch
    q8, k8, w, ks, st, en = _to_dev(case)
    lo = None
    if with_logits:
        lo = torch.full((case.queries, case.keys), float("nan"), dtype=torch.float32, device="cuda")
    b, t = binding.indexer_select(q8, k8, w, ks, st, en, case.block_size, case.k_blocks,
                                  case.k_tokens, case.starts_repeat, case.ends_repeat,
                                  logits_out=lo)
    torch.cuda.synchronize()
    return b.cpu().numpy(), t.cpu().numpy(), (None if lo is None else lo.cpu().numpy())


def _check(case, rows=None, with_logits=True):
    gb, gt, glog = _run(case, with_logits)
    wb, wt, wlog = io.indexer_select(case.q8, case.k8, case.w, case.kscale, case.starts,
                                     case.ends, case.block_size, case.k_blocks,
                                     case.k_tokens, case.starts_repeat, case.ends_repeat,
                                     rows=rows, return_logits=True)
    rows = range(case.queries) if rows is None else rows
    for r in rows:
        assert np.array_equal(gb[r], wb[r]), f"row {r}: block ids differ at {np.nonzero(gb[r] != wb[r])[0][:8]}"
        assert np.array_equal(gt[r], wt[r]), f"row {r}: token ids differ at {np.nonzero(gt[r] != wt[r])[0][:8]}"
        if with_logits and r in wlog:
            s, e, L = io.dsa_oracle.row_bounds(r, case.starts, case.ends, case.keys,
                                               case.starts_repeat, case.ends_repeat)
            got = glog[r, s:e].view(np.uint32)
            assert np.array_equal(got, wlog[r].view(np.uint32)), f"row {r}: logits differ"
            outside = np.concatenate([glog[r, :s], glog[r, e:]])
            assert np.all(np.isnan(outside)), f"row {r}: logits written outside [start, end)"
    gh.log(f"  indexer: {len(list(rows))} rows bit-exact")
    return gb, gt


def test_indexer_tiny_closed_form_tokens():
    ends = [2048, 1, 7, 8, 9, 1000, 3000, 0]
    case = wl.make_indexer_custom(8, 2048, 64, 128, 8, 32, 256, ends, seed=11)
    _check(case)


def test_indexer_recomputed_token_route():
    """K_blk * B > K_tok: the kept blocks' logits are computed again."""
    ends = [3000, 2999, 2000, 101, 100, 99, 17, 3000]
    case = wl.make_indexer_custom(8, 3000, 64, 128, 8, 64, 100, ends, seed=12)
    _check(case)


@pytest.mark.parametrize("H,B,kb,kt", [(16, 1, 200, 150), (32, 2, 100, 200), (64, 4, 50, 200),
                                       (16, 16, 20, 320), (32, 16, 40, 100), (64, 8, 512, 4096),
                                       # either side of the narrow form's limit (384):
                                       # narrow with the recompute route at 384 tokens, wide
                                       # with 385 blocks and with 385 recomputed tokens
                                       (64, 2, 384, 384), (32, 2, 385, 1000), (16, 4, 200, 385)])
def test_indexer_shapes(H, B, kb, kt):
    rng = np.random.default_rng(H * 100 + B)
    Q, S = 6, 9000
    ends = rng.integers(1, S + 50, size=Q)
    starts = rng.integers(0, 2000, size=Q)
    case = wl.make_indexer_custom(Q, S, H, 128, B, kb, kt, ends, starts=starts, seed=H + B)
    _check(case)


def test_indexer_repeats_and_no_key_scale():
    case = wl.make_indexer_custom(8, 5000, 64, 128, 8, 40, 200, [5000, 4000, 3333, 10],
                                  starts=[0, 17], starts_repeat=4, ends_repeat=2,
                                  with_kscale=False, seed=13)
    _check(case)


def test_indexer_long_rows_refill_the_buffer():
    """Rows of 20000-60000 keys (2500-7500 blocks of 8) refill the 1024-entry
    candidate buffer many times."""
    ends = [60000, 45001, 20000, 33333]
    case = wl.make_indexer_custom(4, 60000, 64, 128, 8, 256, 2048, ends, seed=14)
    _check(case)


def test_indexer_rising_row():
    """Keys grow along the row in 24 equal steps (every block beats the
    running threshold, and blocks tie within a step): the kept blocks are
    the lowest ids of the top steps plus the newest block."""
    S = 60000
    level = np.minimum(np.arange(S) // 2500, 23)
    codes = (((5 + level // 8) << 3) | (level % 8)).astype(np.uint8)
    case = wl.make_indexer_custom(3, S, 64, 128, 8, 256, 2048, [S, S - 5, 41000], seed=16)
    case.k8[:] = codes[:, None]
    case.q8[:] = 0x38                                 # every query slice 1.0
    case.w[:] = np.abs(case.w)
    _check(case)


def test_indexer_all_equal_logits():
    """Zero queries: every logit is 0, every block ties; lower ids win."""
    case = wl.make_indexer_custom(4, 20000, 64, 128, 8, 256, 2048, [20000, 19999, 9000, 2049],
                                  seed=15)
    case.q8[:] = 0
    gb, gt = _check(case)
    assert gb[0, :255].tolist() == list(range(255)) and gb[0, 255] == 2499


def test_indexer_small_config_every_row():
    case = wl.make_indexer_config("indexer_small")
    gh.log(f"indexer_small: Q={case.queries} S={case.keys}")
    _check(case, with_logits=False)


def test_indexer_prefill_config_sampled_rows():
    case = wl.make_indexer_config("indexer_prefill")
    rows = [0, 1, 4095, case.queries - 1]
    gh.log(f"indexer_prefill: Q={case.queries} S={case.keys}, oracle rows {rows}")
    _check(case, rows=rows, with_logits=False)


def _indexer_fuzz_case(seed):
    rng = np.random.default_rng(7000 + seed)
    Q = int(rng.choice([1, 3, 8, 13]))
    S = int(rng.integers(1, 20000))
    H = int(rng.choice([16, 32, 64]))
    B = int(rng.choice([1, 2, 4, 8, 16]))
    kb = int(rng.integers(1, 513))
    kt = int(rng.integers(1, 513)) if kb * B > 512 else int(rng.integers(1, 4097))
    sr = int(rng.choice([1, 1, 2]))
    er = int(rng.choice([1, 1, 2]))
    ends = rng.integers(0, S + 30, size=-(-Q // er))
    starts = rng.integers(0, max(1, S // 2), size=-(-Q // sr)) if rng.random() < 0.6 else None
    return wl.make_indexer_custom(Q, S, H, 128, B, kb, kt, ends, starts=starts, seed=seed,
                                  with_kscale=bool(rng.random() < 0.8), starts_repeat=sr,
                                  ends_repeat=er)


@pytest.mark.parametrize("seed", range(16))
def test_indexer_fuzz(seed):
    """Random shapes: 1-13 queries, up to 20,000 keys, 16/32/64 heads, block
    sizes 1-16, K_blk up to 512 (both forms), both token routes, starts,
    repeats, with and without key scales; every row bit for bit."""
    case = _indexer_fuzz_case(seed)
    gh.log(f"indexer fuzz seed={seed} Q={case.queries} S={case.keys} B={case.block_size} "
           f"kb={case.k_blocks} kt={case.k_tokens}")
    _check(case)


@pytest.mark.parametrize("kb,kt", [(32, 256), (64, 100)], ids=["closed_form", "recompute"])
def test_indexer_graph_replay_with_new_ends(kb, kt):
    """A captured indexer call replayed with new ends (the launch shape is
    fixed by the shape; trip counts follow the ends on the device): every
    replay equals the oracle on the new bounds, and five replays of the same
    ends agree bit for bit."""
    import dataclasses
    import torch
    S = 6000
    case = wl.make_indexer_custom(8, S, 64, 128, 8, kb, kt, [S] * 8, seed=15 + kb)
    q8, k8, w, ks, st, en = _to_dev(case)
    bids = torch.empty((case.queries, kb), dtype=torch.int32, device="cuda")
    tids = torch.empty((case.queries, kt), dtype=torch.int32, device="cuda")
    call = lambda: binding.indexer_select(q8, k8, w, ks, st, en, case.block_size, kb, kt,
                                          block_ids=bids, token_ids=tids)
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for new in ([S, 1, 4097, 0, 2500, 17, S - 1, 3000], [9, 9, 9, 9, S, S, 100, 101]):
        ends = np.asarray(new, np.int32)
        en.copy_(torch.from_numpy(ends))
        outs = []
        for _ in range(5):
            bids.fill_(-7)
            tids.fill_(-7)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            outs.append((bids.cpu().numpy(), tids.cpu().numpy()))
        for b, t in outs[1:]:
            assert np.array_equal(b, outs[0][0]) and np.array_equal(t, outs[0][1])
        c2 = dataclasses.replace(case, ends=ends)
        wb, wt, _ = io.indexer_select(c2.q8, c2.k8, c2.w, c2.kscale, c2.starts, c2.ends,
                                      c2.block_size, kb, kt, c2.starts_repeat, c2.ends_repeat,
                                      return_logits=True)
        assert np.array_equal(outs[0][0], wb), f"block ids differ for ends {new}"
        assert np.array_equal(outs[0][1], wt), f"token ids differ for ends {new}"
    gh.log(f"  indexer graph: replays with new ends bit-exact (kb={kb}, kt={kt})")


def test_indexer_rejects_unsupported_shapes():
    import torch
    case = wl.make_indexer_custom(2, 100, 64, 128, 8, 4, 16, [100, 50], seed=1)
    q8, k8, w, ks, st, en = _to_dev(case)
    with pytest.raises(binding.DsaError):
        binding.indexer_select(q8, k8, w, ks, st, en, 3, 4, 16)         # block size 3
    with pytest.raises(binding.DsaError):
        binding.indexer_select(q8, k8, w, ks, st, en, 8, 600, 16)       # k_blocks > 512
    with pytest.raises(binding.DsaError):
        binding.indexer_select(q8, k8, w, ks, st, en, 8, 100, 700)      # recompute, k_tokens > 512
    torch.cuda.synchronize()
