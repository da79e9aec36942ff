"""The decode chain end to end (needs an MI355X): FP8 indexer logits and the
selection in one call (dsa_indexer_select), then the sparse attention over the
selected tokens (dsa_sparse_attn), against the two oracles chained the same
way.

All requests' indexer keys and K/V rows live in one array each, request i at
positions [start_i, end_i) (its rows' live range), so the token ids the
selection returns are absolute positions and index the flat K/V cache
directly (no page table).  The selection is compared bit for bit; the
attention within the bound derived in tests/test_gpu_sparse_attn.py.
"""
import numpy as np
import pytest

from oracle import indexer_oracle as io
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


@pytest.mark.parametrize("B,kb,kt,union", [(8, 64, 512, False), (16, 16, 200, False),
                                            (8, 64, 512, True)])
def test_indexer_selection_then_attention(B, kb, kt, union):
    import torch
    rng = np.random.default_rng(B + kb)
    lens = np.array([6000, 1500, 300, 9000])           # per request
    rows_per_req = 4
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    S = int(lens.sum())
    # row j of request i sees the first len_i - (3 - j) positions of it
    ends = np.array([starts[i] + lens[i] - (rows_per_req - 1 - j)
                     for i in range(lens.size) for j in range(rows_per_req)], np.int32)
    Q = ends.size
    ic = wl.make_indexer_custom(Q, S, 64, 128, B, kb, kt, ends, starts=starts,
                                starts_repeat=rows_per_req, seed=31 + B)
    d = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    _, tok = binding.indexer_select(d(ic.q8), d(ic.k8), d(ic.w), d(ic.kscale), d(ic.starts),
                                    d(ic.ends), B, kb, kt, rows_per_req, 1)
    torch.cuda.synchronize()
    wb, wt = io.indexer_select(ic.q8, ic.k8, ic.w, ic.kscale, ic.starts, ic.ends, B, kb, kt,
                               rows_per_req, 1)
    got_tok = tok.cpu().numpy()
    assert np.array_equal(got_tok, wt), "selected tokens differ from the oracle"

    # attention of each row over its selected tokens, flat cache (slot = position);
    # in union mode the 4 rows of a request run over the union of their ids
    # (groups of 4 rows need 4 * G <= 16 (row, head) pairs, so G = 3)
    hkv, G, D = (2, 3, 128) if union else (2, 6, 128)
    ac = wl.make_attn_custom([S], 1, hkv, G, D, kt, paged=False, seed=41 + B, q_scale=2.0)
    q = wl.bf16_bits(rng.standard_normal((Q, hkv * G, D), dtype=np.float32) * np.float32(2.0))
    gate = wl.bf16_bits(rng.standard_normal((Q, hkv * G, D), dtype=np.float32))
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
        torch.bfloat16).cuda()
    op = binding.SparseAttn(Q, hkv, G, D, kt, ac.num_slots, rows_per_seq=4 if union else 1,
                            union_rows=4 if union else 0)
    out = op(bf(q), bf(ac.k_cache), bf(ac.v_cache), tok, None, bf(gate), ac.sm_scale)
    torch.cuda.synchronize()
    assert op.read_status() == 0
    op.close()
    got = (out.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(
        np.float32).astype(np.float64)
    ref, _, bad = so.sparse_attention(q, ac.k_cache, ac.v_cache, wt, ac.sm_scale, G, gate=gate,
                                      distinct=union)
    A, _, _ = so.sparse_attention(q, ac.k_cache, ac.v_cache & np.uint16(0x7FFF), wt,
                                  ac.sm_scale, G, gate=gate, distinct=union)
    assert bad.sum() == 0
    tol = 2.0 ** -7 * A + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"worst excess {np.max(err - tol):.3e}"
    gh.log(f"  chain: {Q} rows over {S} keys, B={B}, top-{kb} blocks, top-{kt} tokens, "
           f"then attention {hkv}x{G}x{D}{' in union mode' if union else ''}")
