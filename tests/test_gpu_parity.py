"""Parity of the HIP library with the CPU oracle (needs an MI355X).

Every comparison is bit-exact: indices, scores and the masked buffer
(including the tail past end, the head before start and the interleaved
elements of a strided view).  Every row of every case, the full-size
workloads included, is compared with the C oracle (threshold selection, all
host cores); small cases and sampled rows of the full-size workloads are
also compared with the numpy oracle (full sort), and every fused call must
leave the context's status word at zero.
"""
import numpy as np
import pytest

import oracle
from sparse_attention_indexer_start_amd import binding
from sparse_attention_indexer_start_amd import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    binding.load()          # raises if the library is missing: no fallback
    yield
    torch.cuda.synchronize()


def _full_check(dc, bids, tids, scores, write_mask=True):
    gh.check_rows_against_oracle(dc, range(dc.sh.rows), bids, tids, scores, masked=write_mask)
    gh.check_all_rows_c(dc, bids, tids, scores, write_mask)
    gh.check_whole_buffer(dc, write_mask)
    gh.check_invariants_all_rows(dc, bids, tids)


# ---------------------------------------------------------------------------
# Small cases, every row
# ---------------------------------------------------------------------------

def test_fused_tiny_config():
    dc = gh.DevCase(wl.make_config("tiny"))
    gh.log(f"tiny: ends={dc.case.ends.tolist()}")
    bids, tids, scores = dc.run_fused()
    _full_check(dc, bids, tids, scores)


def _fuzz_case(seed):
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.integers(1, 8))
    B = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 32, 64, 128]))
    W = int(rng.integers(1, 6000 if B > 2 else 9000))
    nb = -(-W // B)
    kb = int(rng.choice([1, 2, 7, max(1, nb // 3), nb, nb + 5, 64, 256]))
    kt = int(rng.choice([1, 3, 100, max(1, W // 5), W, W + 3, 2048]))
    cs = int(rng.choice([1, 2]))
    ends = rng.integers(0, W + 40, size=R)
    ends[rng.random(R) < 0.3] = W
    starts = None
    if rng.random() < 0.6:
        starts = rng.integers(0, max(1, W // 2), size=R)
    return wl.make_custom(R, W, B, kb, kt, ends, starts=starts, col_stride=cs,
                          seed=seed, dup_frac=0.1)


@pytest.mark.parametrize("seed", range(24))
def test_fused_fuzz(seed):
    case = _fuzz_case(seed)
    sh = case.shape
    gh.log(f"fuzz seed={seed} R={sh.rows} W={sh.width} B={sh.block_size} "
           f"kb={sh.k_blocks} kt={sh.k_tokens} cs={sh.col_stride} ends={case.ends.tolist()} "
           f"starts={None if case.starts is None else case.starts.tolist()}")
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused()
    _full_check(dc, bids, tids, scores)


def _long_fuzz_case(seed):
    rng = np.random.default_rng(5000 + seed)
    R = int(rng.choice([1, 2, 5, 17, 40, 130, 300]))
    B = int(rng.choice([1, 2, 4, 8, 16, 32]))
    W = int(rng.integers(20000, 400000 if R <= 40 else 60000))
    nb = -(-W // B)
    kb = int(rng.choice([1, 5, 64, 300, 2048, min(nb, 8000)]))
    kt = int(rng.choice([1, 100, 2048, 5000]))
    kb = min(kb, 65536 - kt)
    cs = int(rng.choice([1, 2]))
    ends = rng.integers(0, W + 100, size=R)
    ends[rng.random(R) < 0.25] = W
    starts = rng.integers(0, W // 3, size=R) if rng.random() < 0.5 else None
    return wl.make_custom(R, W, B, kb, kt, ends, starts=starts, col_stride=cs, seed=seed,
                          dup_frac=0.02, outlier_frac=0.01)


@pytest.mark.parametrize("seed", range(40))
def test_fused_long_fuzz(seed):
    """Random shapes with long rows: 1 to 300 rows (balanced and per-row
    splits), widths up to 400,000, block sizes 1 to 32, K from 1 to 8000,
    strided views and starts, in one launch or two."""
    case = _long_fuzz_case(seed)
    sh = case.shape
    two = bool(seed % 3 == 2)
    gh.log(f"long fuzz seed={seed} R={sh.rows} W={sh.width} B={sh.block_size} kb={sh.k_blocks} "
           f"kt={sh.k_tokens} cs={sh.col_stride} starts={'yes' if case.starts is not None else 'no'} "
           f"two_launches={two}")
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused(two_launches=two)
    rows = range(min(sh.rows, 8))
    gh.check_rows_against_oracle(dc, rows, bids, tids, scores)
    gh.check_all_rows_c(dc, bids, tids, scores)
    gh.check_whole_buffer(dc)
    gh.check_invariants_all_rows(dc, bids, tids)


@pytest.mark.parametrize("two", [False, True], ids=["one_launch", "two_launches"])
@pytest.mark.parametrize("B,W,ends,kb,kt", [
    (8, 65536, [65536, 40000, 16385], 16, 100),
    (8, 65536, [65536, 40000, 16385], 1000, 2048),
    (8, 65536, [65536, 40001, 16399], 3000, 9000),
    (1, 12000, [12000, 4097, 2049, 11999], 50, 70),
    (2, 30000, [30000, 20001, 4097], 2047, 5000),
    (16, 140000, [140000, 70000, 32769], 128, 2048),
    (8, 300000, [300000, 299999, 150001, 65537], 2048, 2048),
    (16, 65536, [65536, 30000, 16385, 16384], 128, 2048),   # medium rows: split
    (8, 32768, [32768, 16385, 16384, 20001], 300, 3000),
    (4, 200000, [200000, 100003], 600, 5000),
    (64, 40000, [40000, 30001, 16385], 700, 3000),          # medium rows, every block kept
])
def test_fused_long_rows(B, W, ends, kb, kt, two):
    """Rows longer than one workgroup's LDS share: the two-pass path."""
    case = wl.make_custom(len(ends), W, B, kb, kt, ends, seed=B * 7 + kb, dup_frac=0.02,
                          outlier_frac=0.01)
    gh.log(f"long rows B={B} W={W} ends={ends} kb={kb} kt={kt} two_launches={two}")
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused(two_launches=two)
    _full_check(dc, bids, tids, scores)


@pytest.mark.parametrize("with_scores", [True, False], ids=["scores", "no_scores"])
def test_fused_medium_rows_keep_all(with_scores):
    """Rows of at most LIST_CAP blocks that are longer than one workgroup
    reads alone (the two-pass split), with K_blk at or above their block
    count: every block is kept, with and without a scores output."""
    ends = [65536, 40000, 16385, 16384, 30000]
    case = wl.make_custom(len(ends), 65536, 32, 2048, 3000, ends, seed=313, dup_frac=0.05)
    gh.log(f"medium rows keep all ends={ends} with_scores={with_scores}")
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused(with_scores=with_scores)
    gh.check_rows_against_oracle(dc, range(dc.sh.rows), bids, tids, scores)
    gh.check_all_rows_c(dc, bids, tids, scores)
    gh.check_whole_buffer(dc)


@pytest.mark.parametrize("two", [False, True], ids=["one_launch", "two_launches"])
def test_fused_medium_rows_per_row_split(two):
    """300 rows take the per-row split with two workgroups per row: rows of at
    most LIST_CAP blocks but longer than one workgroup reads alone go through
    both passes and the final workgroup, in one launch and in two."""
    rng = np.random.default_rng(4242)
    R, W = 300, 32768
    ends = rng.integers(16385, W + 1, size=R)
    ends[:8] = [W, 16385, 16384, 1, 0, 20000, W - 1, 30001]
    starts = rng.integers(0, 64, size=R)
    case = wl.make_custom(R, W, 8, 300, 3000, ends, starts=starts, col_stride=2 if two else 1,
                          seed=4242, dup_frac=0.02, outlier_frac=0.01)
    gh.log(f"medium rows per-row split R={R} W={W} two_launches={two}")
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused(two_launches=two)
    _full_check(dc, bids, tids, scores)


@pytest.mark.parametrize("value", [1.5, -2.0])
def test_fused_long_rows_all_ties(value):
    """Long rows whose live values are all equal: every block ties, so every
    block is listed and every value is a token candidate (the per-piece
    candidate space overflows); ties go to the lower index."""
    ends = [40000, 20000, 16385]
    case = wl.make_custom(len(ends), 40000, 8, 300, 1000, ends, seed=91)
    for r, e in enumerate(ends):
        case.logits[r, :e] = np.float32(value)
    gh.log(f"long rows all ties value={value}")
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused()
    _full_check(dc, bids, tids, scores)


def test_fused_long_rows_with_start_and_stride():
    case = wl.make_custom(4, 50000, 8, 300, 2048, [50000, 49999, 30000, 45000],
                          starts=[0, 7, 1001, 44990], col_stride=2, seed=77, dup_frac=0.05)
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused()
    _full_check(dc, bids, tids, scores)


def test_fused_large_k_blocks():
    """K_blk = 100000 of 131072 blocks: the count of keys above the digit's bin
    needs 17 bits of the row's ready word."""
    ends = [1048576, 900001]
    case = wl.make_custom(len(ends), 1048576, 8, 100000, 2048, ends, seed=5, dup_frac=0.01)
    gh.log(f"large k_blocks ends={ends}")
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused()
    _full_check(dc, bids, tids, scores)


def test_fused_long_rows_concentrated_lists():
    """Sixteen long rows; in the even ones the values rise along the row, so
    every kept block lies in the row's last pieces (more listed entries per
    piece than the final workgroup's per-piece share: the general gather),
    while the odd rows are random (the one-round-trip gather)."""
    W = 262144
    ends = [W, W - 3, 200001, W, 150000, W - 8, W, 131073] * 2
    case = wl.make_custom(len(ends), W, 8, 2048, 2048, ends, seed=23, outlier_frac=0.01)
    for r in range(0, len(ends), 2):
        e = ends[r]
        case.logits[r, :e] = np.linspace(-3.0, 3.0, e, dtype=np.float32)
    gh.log(f"concentrated lists ends={ends}")
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused()
    _full_check(dc, bids, tids, scores)


@pytest.mark.parametrize("W,B,kb,kt", [(3000, 8, 40, 300), (5000, 4, 300, 2048),
                                       (70000, 8, 600, 2048), (40000, 16, 64, 4000)])
def test_fused_special_values(W, B, kb, kt):
    """-inf, +inf, -0 and NaN bit patterns inside the live span.

    They are outside the input contract, but the order key still defines the
    result (NaNs rank by their bits; +inf blocks can tie with the pinned one),
    and the library must reproduce the oracle exactly."""
    ends = [W, W - 7, W // 2 + 3, W // 3]
    case = wl.make_custom(len(ends), W, B, kb, kt, ends, seed=W + B, dup_frac=0.05)
    rng = np.random.default_rng(W)
    specials = np.array([0xFF800000, 0x7F800000, 0x80000000, 0x7FC00000, 0xFFC00001],
                        dtype=np.uint32)
    u = case.buf.view(np.uint32)
    for r, e in enumerate(ends):
        pos = rng.choice(min(e, W), size=max(1, min(e, W) // 50), replace=False)
        u[r, pos] = rng.choice(specials, size=pos.size)
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused()
    gh.check_rows_against_oracle(dc, range(dc.sh.rows), bids, tids, scores)


def test_fused_without_mask_leaves_buffer():
    case = wl.make_custom(4, 40000, 8, 64, 500, [40000, 100, 20000, 3], seed=5)
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused(write_mask=False)
    _full_check(dc, bids, tids, scores, write_mask=False)


def test_fused_repeatable():
    case = wl.make_custom(3, 70000, 8, 500, 3000, [70000, 33000, 9000], seed=9, dup_frac=0.05)
    dc = gh.DevCase(case)
    ctx = dc.context()
    first = None
    for i in range(4):
        dc.restore()
        out = [t.cpu().numpy().copy() for t in dc.run_fused(ctx)[:2]]
        if first is None:
            first = out
        else:
            assert all(np.array_equal(a, b) for a, b in zip(first, out)), f"run {i} differs"
    ctx.close()


@pytest.mark.parametrize("name", ["long_rows", "short_rows"])
def test_graph_replays_bit_identical(name):
    """One captured fused call replayed 100 times, the buffer restored by
    eager copies between replays: every replay equals the first, which equals
    the C oracle, and the status word stays zero."""
    import torch
    if name == "long_rows":
        case = wl.make_custom(4, 300000, 8, 2048, 2048, [300000, 299999, 150001, 65537],
                              seed=17, dup_frac=0.02, outlier_frac=0.01)
    else:
        case = wl.make_custom(6, 20000, 8, 256, 2048, [20000, 8192, 4000, 2049, 300, 1],
                              seed=18, dup_frac=0.02)
    dc = gh.DevCase(case)
    ctx = dc.context()
    bids, tids, scores = dc.outputs()
    ctx.select_fused(dc.logits, dc.starts, dc.ends, bids, tids, scores, True)
    torch.cuda.synchronize()
    dc.restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ctx.select_fused(dc.logits, dc.starts, dc.ends, bids, tids, scores, True)
    torch.cuda.synchronize()
    ref = None
    for i in range(100):
        dc.restore()
        bids.fill_(-7)
        tids.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (bids.cpu().numpy(), tids.cpu().numpy(), scores.cpu().numpy().view(np.uint32),
               dc.buf.cpu().numpy().view(np.uint32))
        if ref is None:
            ref = got
            gh.check_all_rows_c(dc, bids, tids, scores)
        else:
            for a, b in zip(ref, got):
                assert np.array_equal(a, b), f"replay {i} differs from the first"
    gh.assert_status_clean(ctx)
    ctx.close()


def test_width_independence_short_decode():
    """The short-decode rows at widths 8192 and 1,048,576: same outputs (and
    both equal the C oracle); the kernel time is logged for both."""
    import torch
    outs = {}
    for W in (8192, 1048576):
        case = wl.make_config("short_decode", width=W)
        dc = gh.DevCase(case)
        ctx = dc.context()
        bids, tids, _ = dc.run_fused(ctx, with_scores=False)
        gh.check_all_rows_c(dc, bids, tids, None)
        outs[W] = (bids.cpu().numpy(), tids.cpu().numpy(),
                   dc.buf[:, :8192].cpu().numpy().view(np.uint32))
        # time 20 calls on restored copies (HIP events on the launch stream)
        copies = [dc.pristine.clone() for _ in range(20)]
        stream = torch.cuda.current_stream()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for c in copies:
            ctx.select_fused(c, dc.starts, dc.ends, bids, tids, None, True)
        e1.record(stream)
        torch.cuda.synchronize()
        gh.assert_status_clean(ctx)
        gh.log(f"width {W}: {e0.elapsed_time(e1) / 20 * 1e3:.2f} us per eager call, "
               f"grid {ctx.info().grid_groups} workgroups")
        ctx.close()
        del copies, dc
    a, b = outs[8192], outs[1048576]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# The four steps one by one
# ---------------------------------------------------------------------------

def _run_steps(dc):
    import torch
    sh = dc.sh
    ctx = dc.context()
    dev = dc.buf.device
    scores = torch.full((sh.rows, sh.nblocks), gh.SCORE_FILL_BITS, dtype=torch.int32,
                        device=dev).view(torch.float32)
    ctx.block_scores(dc.logits, dc.starts, dc.ends, scores)
    bids = torch.full((sh.rows, sh.k_blocks), 777, dtype=torch.int32, device=dev)
    ctx.topk_blocks(scores, dc.starts, dc.ends, bids)
    tids_virtual = torch.full((sh.rows, sh.k_tokens), 777, dtype=torch.int32, device=dev)
    ctx.topk_tokens(dc.logits, dc.starts, dc.ends, bids, tids_virtual)
    ctx.candidate_mask(dc.logits, dc.starts, dc.ends, bids)
    tids_plain = torch.full((sh.rows, sh.k_tokens), 777, dtype=torch.int32, device=dev)
    ctx.topk_tokens(dc.logits, dc.starts, dc.ends, None, tids_plain)
    torch.cuda.synchronize()
    ctx.close()
    return scores, bids, tids_virtual, tids_plain


@pytest.mark.parametrize("which", ["tiny", "fuzz3", "fuzz8", "long"])
def test_steps_match_oracle(which):
    if which == "tiny":
        case = wl.make_config("tiny")
    elif which == "long":
        case = wl.make_custom(3, 65536, 8, 700, 2500, [65536, 30001, 17000], seed=4,
                              dup_frac=0.03)
    else:
        case = _fuzz_case(int(which[4:]))
    dc = gh.DevCase(case)
    scores, bids, tv, tp = _run_steps(dc)
    # scores/ids/mask/tokens equal the fused chain's, which the oracle defines
    gh.check_rows_against_oracle(dc, range(dc.sh.rows), bids, tv, scores)
    gh.check_rows_against_oracle(dc, range(dc.sh.rows), bids, tp, scores)
    gh.check_whole_buffer(dc)


def test_plain_row_topk_matches_oracle():
    case = wl.make_custom(5, 20000, 8, 1, 1500, [20000, 1, 1499, 1501, 12345],
                          starts=[0, 0, 3, 0, 10], seed=12, dup_frac=0.1)
    dc = gh.DevCase(case)
    import torch
    ctx = dc.context()
    out = torch.empty((5, 1500), dtype=torch.int32, device=dc.buf.device)
    ctx.topk_tokens(dc.logits, dc.starts, dc.ends, None, out)
    torch.cuda.synchronize()
    ctx.close()
    want = oracle.topk_tokens(case.logits, case.starts, case.ends, 8, 1500)
    assert np.array_equal(out.cpu().numpy(), want)


def test_mask_with_unsorted_and_invalid_ids():
    """The mask takes ids in any order; -1 and out-of-range ids are ignored."""
    import torch
    case = wl.make_custom(2, 5000, 8, 6, 10, [5000, 333], seed=2)
    dc = gh.DevCase(case)
    ids = np.array([[600, 3, -1, 624, 10**6, 3], [41, 0, -7, 2, 1, 50]], dtype=np.int32)
    ctx = dc.context()
    ctx.candidate_mask(dc.logits, dc.starts, dc.ends, torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    ctx.close()
    want = oracle.candidate_mask(case.logits, case.starts, case.ends, 8, ids)
    got = dc.logits.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------------------
# The pages' edge lists (report on vllm PR #56628, test code)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("width", [8192, 262144])
@pytest.mark.parametrize("col_stride", [1, 2])
@pytest.mark.parametrize("B", [8, 16])
def test_page_ragged_ends(width, col_stride, B):
    ends = [0, 1, 1023, 1024, 1025, width - 1, width, width // 2]
    case = wl.make_custom(len(ends), width, B, 64, 1024, ends, col_stride=col_stride,
                          seed=width + B + col_stride)
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused()
    _full_check(dc, bids, tids, scores)


def test_page_sentinel_tail_untouched():
    """Buffer filled with 1.5: every value ties; the tail past end stays 1.5."""
    import torch
    W = 262144
    ends = [0, 1, 1025, W // 2]
    case = wl.make_custom(len(ends), W, 8, 64, 1024, ends, seed=3)
    case.buf[:] = np.float32(1.5)
    dc = gh.DevCase(case)
    bids, tids, scores = dc.run_fused()
    _full_check(dc, bids, tids, scores)
    buf = dc.buf.cpu().numpy()
    for r, e in enumerate(ends):
        assert np.all(buf[r, e:] == np.float32(1.5))


def test_graph_replay_tracks_changing_ends():
    """Capture once at one set of ends, replay with others (wide width)."""
    import torch
    W = 262144
    captured = [1024, 4096, 8192, 2048]
    replays = [[1, 131072, W, 0], [W, 1025, 3, 65536], [5000, 0, 262143, 70001]]
    full = wl.make_custom(4, W, 8, 256, 2048, [W] * 4, seed=21, dup_frac=0.01)
    dc = gh.DevCase(full)
    dc.ends.copy_(torch.tensor(captured, dtype=torch.int32))
    ctx = dc.context()
    bids, tids, scores = dc.outputs()
    # first call outside the graph
    ctx.select_fused(dc.logits, dc.starts, dc.ends, bids, tids, scores, True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ctx.select_fused(dc.logits, dc.starts, dc.ends, bids, tids, scores, True)
    torch.cuda.synchronize()
    for rep in range(2):
        for ends in replays:
            gh.log(f"replay {rep} ends={ends}")
            dc.restore()
            dc.ends.copy_(torch.tensor(ends, dtype=torch.int32))
            scores.view(torch.int32).fill_(gh.SCORE_FILL_BITS)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            case = wl.Case("replay", full.shape, full.buf, None, np.array(ends, np.int32), 21)
            dcv = gh.DevCase.__new__(gh.DevCase)
            dcv.case, dcv.sh, dcv.buf, dcv.pristine = case, case.shape, dc.buf, dc.pristine
            dcv.starts, dcv.ends = None, dc.ends
            _full_check(dcv, bids, tids, scores)
            gh.assert_status_clean(ctx)
    ctx.close()


def test_negative_start_is_flagged_and_empty():
    import torch
    case = wl.make_custom(3, 1000, 8, 4, 16, [500, 900, 300], starts=[-3, 0, 10], seed=1)
    dc = gh.DevCase(case)
    ctx = dc.context()
    bids, tids, scores = dc.outputs()
    ctx.select_fused(dc.logits, dc.starts, dc.ends, bids, tids, scores, True)
    torch.cuda.synchronize()
    assert ctx.read_status() & 1
    assert np.all(bids.cpu().numpy()[0] == -1) and np.all(tids.cpu().numpy()[0] == -1)
    gh.check_rows_against_oracle(dc, [1, 2], bids, tids, scores)
    ctx.reset_workspace()
    torch.cuda.synchronize()
    assert ctx.read_status() == 0
    ctx.close()


def test_empty_shapes_are_noops():
    import torch
    for rows, width in ((0, 100), (3, 0)):
        ctx = binding.Context(rows, width, 8, 4, 4)
        lg = torch.zeros((rows, width), dtype=torch.float32, device="cuda")
        e = torch.zeros((max(rows, 1),), dtype=torch.int32, device="cuda")
        b = torch.zeros((rows, 4), dtype=torch.int32, device="cuda")
        t = torch.zeros((rows, 4), dtype=torch.int32, device="cuda")
        ctx.select_fused(lg, None, e, b, t)
        ctx.close()
    torch.cuda.synchronize()


def test_binding_rejects_mismatched_tensors():
    import torch
    ctx = binding.Context(4, 100, 8, 4, 4)
    lg = torch.zeros((4, 100), dtype=torch.float32, device="cuda")
    e = torch.zeros((4,), dtype=torch.int32, device="cuda")
    b = torch.zeros((4, 4), dtype=torch.int32, device="cuda")
    t = torch.zeros((4, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        ctx.select_fused(lg.double(), None, e, b, t)
    with pytest.raises(ValueError):
        ctx.select_fused(lg, None, e.long(), b, t)
    with pytest.raises(ValueError):
        ctx.select_fused(lg[:, :50], None, e, b, t)
    with pytest.raises(ValueError):
        ctx.select_fused(lg, None, e, b[:, :2].contiguous(), t)
    ctx.close()


# ---------------------------------------------------------------------------
# The five workloads at full size (the launch configuration bench.py times)
# ---------------------------------------------------------------------------

def _sample_rows(case, n_random=6, seed=0):
    sh = case.shape
    L = np.array([oracle.row_bounds(r, case.starts, case.ends, sh.width, sh.starts_repeat,
                                    sh.ends_repeat)[2] for r in range(sh.rows)])
    rows = {0, sh.rows - 1, int(L.argmax()), int(L.argmin())}
    rng = np.random.default_rng(seed)
    rows.update(int(x) for x in rng.choice(sh.rows, size=min(n_random, sh.rows), replace=False))
    return sorted(rows)


@pytest.mark.parametrize("name,two", [
    ("short_decode", False), ("mtp_ragged", False), ("mtp_ragged", True),
    ("long_decode", False), ("long_decode", True), ("prefill_chunk", False)])
def test_full_size_workload(name, two):
    """Every row of the workload, as the bench runs it (no scores) and with
    scores, against the C oracle; sampled rows against the numpy oracle."""
    gh.log(f"workload {name}: generating")
    case = wl.make_config(name)
    dc = gh.DevCase(case)
    gh.log(f"workload {name}: running (two_launches={two}, no scores)")
    bids, tids, _ = dc.run_fused(two_launches=two, with_scores=False)
    gh.check_all_rows_c(dc, bids, tids, None)
    gh.check_whole_buffer(dc)
    rows = _sample_rows(case, n_random=8 if name != "long_decode" else 4)
    if name == "mtp_ragged":
        rows = sorted(set(rows) | set(range(16)))   # the edge requests 1023/1024/1025/width
    gh.log(f"workload {name}: numpy oracle rows {rows}")
    gh.check_rows_against_oracle(dc, rows, bids, tids, None)
    dc.restore()
    gh.log(f"workload {name}: running with scores")
    bids, tids, scores = dc.run_fused(two_launches=two, with_scores=True)
    gh.check_all_rows_c(dc, bids, tids, scores)


def test_prefill_graph_replay_new_ends():
    """Prefill-chunk shape: capture once, replay with the +100/+200 end sets;
    every row of every replay against the C oracle."""
    import torch
    base = wl.make_config("prefill_chunk")
    dc = gh.DevCase(base)
    ctx = dc.context()
    bids, tids, scores = dc.outputs()
    ctx.select_fused(dc.logits, dc.starts, dc.ends, bids, tids, scores, True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ctx.select_fused(dc.logits, dc.starts, dc.ends, bids, tids, scores, True)
    torch.cuda.synchronize()
    for off in (100, 200):
        case = wl.make_config("prefill_chunk", seed_offset=off)
        gh.log(f"prefill replay seed offset {off}")
        dc.buf.copy_(torch.from_numpy(case.buf))
        dc.pristine.copy_(dc.buf)
        dc.ends.copy_(torch.from_numpy(case.ends))
        scores.view(torch.int32).fill_(gh.SCORE_FILL_BITS)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gh.assert_status_clean(ctx)
        dc.case = case
        gh.check_all_rows_c(dc, bids, tids, scores)
        gh.check_whole_buffer(dc)
        gh.check_rows_against_oracle(dc, _sample_rows(case, 6, seed=off), bids, tids, scores)
    ctx.close()
