"""Parity of the cooperative per-row top-k for very long rows (needs an MI355X).

Every row is compared element by element with the numpy oracle's top-k (a
full sort on (value desc, column asc), pinned in tests/oracle_pins.py):
rows of 1..20,000 columns with every k from 1 to beyond the row, ties,
special values, non-zero starts, repeats and a strided view; rows of 4 and
16 million columns with k of 2048 and of a million; a row whose list part
overflows (it falls back to reading the row) and a row settled after the
second digit in list mode; k above the row length; agreement with dsa_topk on
rows of 200,000; graph replay with changed ends.
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
    binding.load()
    yield
    torch.cuda.synchronize()


def _want(lg, starts, ends, k, sr=1, er=1):
    rows, width = lg.shape
    out = np.full((rows, k), -1, np.int32)
    for r in range(rows):
        s, e, L = oracle.row_bounds(r, starts, ends, width, sr, er)
        if L == 0:
            continue
        ids = oracle.top_k_indices(oracle.order_keys(np.asarray(lg[r, s:e], np.float32)), k)
        out[r, : ids.size] = ids + s
    return out


def _run(case_buf, cs, width, starts, ends, k, sr=1, er=1):
    import torch
    buf = torch.from_numpy(case_buf).cuda()
    view = buf[:, ::cs]
    st = None if starts is None else torch.from_numpy(np.asarray(starts, np.int32)).cuda()
    en = torch.from_numpy(np.asarray(ends, np.int32)).cuda()
    op = binding.RowTopk(view.shape[0], width, k, row_stride=view.stride(0), col_stride=cs,
                         starts_repeat=sr, ends_repeat=er)
    out = op(view, st, en)
    torch.cuda.synchronize()
    gh.log(f"  row top-k: {view.shape[0]} rows x {width}, k={k}, {op.pieces()} pieces per row")
    op.close()
    return out.cpu().numpy()


def _check_case(case, k):
    sh = case.shape
    got = _run(case.buf, sh.col_stride, sh.width, case.starts, case.ends, k,
               sh.starts_repeat, sh.ends_repeat)
    want = _want(case.logits, case.starts, case.ends, k, sh.starts_repeat, sh.ends_repeat)
    bad = np.nonzero((got != want).any(1))[0]
    assert bad.size == 0, f"rows {bad[:8]} differ (first at {np.nonzero(got[bad[0]] != want[bad[0]])[0][:8]})"


@pytest.mark.parametrize("seed", range(10))
def test_row_topk_small_fuzz(seed):
    rng = np.random.default_rng(700 + seed)
    R = int(rng.integers(1, 7))
    W = int(rng.integers(1, 20000))
    k = int(rng.choice([1, 7, 300, max(1, W // 3), W, W + 11]))
    cs = int(rng.choice([1, 2]))
    ends = rng.integers(0, W + 30, size=R)
    starts = rng.integers(0, max(1, W // 2), size=R) if rng.random() < 0.5 else None
    case = wl.make_custom(R, W, 8, 1, 1, ends, starts=starts, col_stride=cs, seed=seed,
                          dup_frac=0.2)
    _check_case(case, k)


@pytest.mark.parametrize("seed", range(10))
def test_row_topk_long_fuzz(seed):
    """Random long rows: 1-4 rows of up to 4M columns, K from 1 to 2^20
    (list mode, its overflow fallback and rows read four times), strided
    views, starts, ties and outliers."""
    rng = np.random.default_rng(800 + seed)
    R = int(rng.integers(1, 5))
    W = int(rng.integers(100000, 4 * 2**20))
    k = int(rng.choice([1, 64, 2048, 30000, 2**20]))
    cs = int(rng.choice([1, 1, 2]))
    ends = rng.integers(W // 2, W + 30, size=R)
    starts = rng.integers(0, W // 4, size=R) if rng.random() < 0.5 else None
    case = wl.make_custom(R, W, 8, 1, 1, ends, starts=starts, col_stride=cs, seed=seed,
                          dup_frac=0.05, outlier_frac=0.001)
    gh.log(f"row top-k long fuzz seed={seed} R={R} W={W} k={k} cs={cs}")
    _check_case(case, k)


def test_row_topk_special_values_and_ties():
    W = 30000
    case = wl.make_custom(3, W, 8, 1, 1, [W, W - 1, 12345], seed=3, dup_frac=0.3)
    rng = np.random.default_rng(3)
    u = case.buf.view(np.uint32)
    specials = np.array([0x80000000, 0x00000000, 0xFF800000, 0x7F800000], np.uint32)
    for r in range(3):
        pos = rng.choice(12345, size=2000, replace=False)
        u[r, pos] = rng.choice(specials, size=pos.size)
    case.buf[2, :12345] = np.float32(1.0)            # a row of one value: all ties
    for k in (1, 1000, 12345, 40000):
        _check_case(case, k)


def test_row_topk_repeats():
    case = wl.make_custom(8, 50000, 8, 1, 1, [50000, 30000, 2, 49999], starts=[0, 1000],
                          starts_repeat=4, ends_repeat=2, seed=5)
    _check_case(case, 5000)


@pytest.mark.parametrize("W,k", [(4 * 2**20, 2048), (4 * 2**20, 2**20), (16 * 2**20, 2048),
                                 (16 * 2**20, 2**20)])
def test_row_topk_very_long_rows(W, k):
    ends = [W, W - 12345] if W <= 4 * 2**20 else [W]
    starts = [0, 777] if len(ends) == 2 else None
    case = wl.make_custom(len(ends), W, 8, 1, 1, ends, starts=starts, seed=W // 1000 + k,
                          dup_frac=0.01, outlier_frac=0.001)
    gh.log(f"very long rows W={W} k={k}")
    _check_case(case, k)


def test_row_topk_list_overflow_falls_back():
    """Row 0 holds its 5000 largest values inside its first piece, so that
    piece's list of the first digit's bin and up overflows and the row falls
    back to reading the row; row 1 (ordinary values) runs on its lists."""
    W, k = 4 * 2**20, 2048
    case = wl.make_custom(2, W, 8, 1, 1, [W, W - 3], seed=13)
    rng = np.random.default_rng(13)
    cols = rng.choice(16384, size=5000, replace=False)
    case.buf[0, cols] = (np.float32(100.0) + np.arange(5000, dtype=np.float32) * np.float32(0.01))
    _check_case(case, k)


def test_row_topk_list_mode_settles_on_third_digit():
    """The 1500 largest values share the first digit's bin and have distinct
    second digits, so the K-th key's bin after two digits holds it alone: the
    row is settled before the third digit and counted from its lists."""
    W, k = 2**20, 1000
    case = wl.make_custom(1, W, 8, 1, 1, [W], seed=17)
    rng = np.random.default_rng(17)
    case.buf[0, :] = rng.random(W, dtype=np.float32) * np.float32(0.9)
    cols = rng.choice(W, size=1500, replace=False)
    case.buf[0, cols] = np.float32(1.0) + np.arange(1500, dtype=np.float32) * np.float32(2.0 ** -15)
    _check_case(case, k)


def test_row_topk_many_listed_settles_on_third_digit():
    """8000 large values: 3904 in the first digit's top bin and 4096 in the
    next one, with distinct second digits, and k = 6500: the row is settled
    after two digits with 2596 of the 4096 keys of the second bin taken,
    counted and emitted from lists that span both bins."""
    W, k = 2**20, 6500
    case = wl.make_custom(1, W, 8, 1, 1, [W], seed=19)
    rng = np.random.default_rng(19)
    case.buf[0, :] = rng.random(W, dtype=np.float32) * np.float32(0.9)
    cols = rng.choice(W, size=8000, replace=False)
    case.buf[0, cols] = np.float32(1.0) + np.arange(8000, dtype=np.float32) * np.float32(2.0 ** -15)
    _check_case(case, k)


def test_row_topk_k_beyond_row():
    W = 3 * 2**20
    case = wl.make_custom(2, W, 8, 1, 1, [W, 2 * 2**20], seed=9)
    got = _run(case.buf, 1, W, None, case.ends, 4 * 2**20)
    for r, L in enumerate([W, 2 * 2**20]):
        assert np.array_equal(got[r, :L], np.arange(L, dtype=np.int32))
        assert np.all(got[r, L:] == -1)


def test_row_topk_matches_dsa_topk():
    import torch
    W, k = 200000, 2048
    case = wl.make_custom(8, W, 8, 256, k, [W, 150000, 3000, 2049, 2048, 1, 0, 199999],
                          seed=11, dup_frac=0.05)
    got = _run(case.buf, 1, W, None, case.ends, k)
    dc = gh.DevCase(case)
    ctx = dc.context()
    out = torch.empty((8, k), dtype=torch.int32, device="cuda")
    ctx.topk_tokens(dc.logits, dc.starts, dc.ends, None, out)
    torch.cuda.synchronize()
    ctx.close()
    assert np.array_equal(got, out.cpu().numpy())


def test_row_topk_graph_replay_changing_ends():
    import torch
    W, k = 2**20, 4096
    case = wl.make_custom(3, W, 8, 1, 1, [W, W, W], seed=13, dup_frac=0.02)
    buf = torch.from_numpy(case.buf).cuda()
    ends = torch.tensor([W, 1000, 500000], dtype=torch.int32, device="cuda")
    op = binding.RowTopk(3, W, k)
    out = torch.empty((3, k), dtype=torch.int32, device="cuda")
    op(buf, None, ends, out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op(buf, None, ends, out)
    torch.cuda.synchronize()
    for new in ([1, W, 4096], [W - 1, 300000, 0], [5000, 5000, 5000]):
        ends.copy_(torch.tensor(new, dtype=torch.int32))
        out.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = _want(case.logits, None, np.array(new, np.int32), k)
        assert np.array_equal(out.cpu().numpy(), want), new
    op.close()


def test_row_topk_replays_bit_identical():
    """30 graph replays of a 16M-column row with k = 2^20 (all three digits
    and the suffix-count placement), each equal to the oracle: a check on
    anything that depends on when the pieces of one launch start."""
    import torch
    W, k = 16 * 2**20, 2**20
    case = wl.make_custom(1, W, 8, 1, 1, [W - 3], seed=17, dup_frac=0.02)
    buf = torch.from_numpy(case.buf).cuda()
    ends = torch.from_numpy(case.ends).cuda()
    op = binding.RowTopk(1, W, k)
    out = torch.empty((1, k), dtype=torch.int32, device="cuda")
    op(buf, None, ends, out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op(buf, None, ends, out)
    torch.cuda.synchronize()
    want = _want(case.logits, None, case.ends, k)
    for it in range(30):
        out.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), want), f"replay {it} differs"
    op.close()
