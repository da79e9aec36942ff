"""The allocation-free entry point against the context entry point (GPU).

Two calls in a row through dsa_select_fused_noalloc, the second with a
smaller input of another shape, each compared bit for bit with
dsa_select_fused on a context of the same shape: block ids, token ids,
scores and the whole masked buffer; the caller's status word stays zero.
"""
import numpy as np
import pytest

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


def _run_both(case):
    import torch
    sh = case.shape
    gh.log(f"no-alloc: rows={sh.rows} width={sh.width} B={sh.block_size} kb={sh.k_blocks} "
           f"kt={sh.k_tokens} cs={sh.col_stride}")
    a = gh.DevCase(case)
    b = gh.DevCase(case)
    want_b, want_t, want_s = a.outputs()
    ctx = a.context()
    ctx.select_fused(a.logits, a.starts, a.ends, want_b, want_t, want_s, True)
    torch.cuda.synchronize()
    gh.assert_status_clean(ctx)
    ctx.close()
    got_b, got_t, got_s = b.outputs()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.select_fused_noalloc(b.logits, b.starts, b.ends, got_b, got_t, sh.block_size,
                                 sh.k_blocks, sh.k_tokens, scores=got_s, write_mask=True,
                                 starts_repeat=sh.starts_repeat, ends_repeat=sh.ends_repeat,
                                 status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(got_b.cpu().numpy(), want_b.cpu().numpy())
    assert np.array_equal(got_t.cpu().numpy(), want_t.cpu().numpy())
    assert np.array_equal(got_s.cpu().numpy().view(np.uint32), want_s.cpu().numpy().view(np.uint32))
    assert np.array_equal(b.buf.cpu().numpy().view(np.uint32), a.buf.cpu().numpy().view(np.uint32))
    return b, got_b, got_t, got_s


def test_noalloc_matches_context_entry_point_twice():
    big = wl.make_custom(8, 262144, 8, 2048, 2048,
                         [262144, 262143, 200001, 150000, 70000, 9000, 300, 0],
                         starts=[0, 5, 17, 1000, 0, 3, 0, 0], seed=31, dup_frac=0.02,
                         outlier_frac=0.01)
    _run_both(big)
    small = wl.make_custom(4, 40000, 16, 128, 2048, [40000, 20000, 33, 39999],
                           starts=[0, 7], starts_repeat=2, col_stride=2, seed=32,
                           dup_frac=0.02)
    dc, b, t, s = _run_both(small)
    gh.check_all_rows_c(dc, b, t, s)


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    import torch
    rows, width = 2048, 131072   # block keys and lists alone need about 537 MB
    lg = torch.empty((rows, width), dtype=torch.float32, device="cuda")
    e = torch.zeros(rows, dtype=torch.int32, device="cuda")
    b = torch.empty((rows, 256), dtype=torch.int32, device="cuda")
    t = torch.empty((rows, 2048), dtype=torch.int32, device="cuda")
    with pytest.raises(binding.DsaError) as ei:
        binding.select_fused_noalloc(lg, None, e, b, t, 8, 256, 2048)
    assert ei.value.code == -2 and "workspace" in str(ei.value)
