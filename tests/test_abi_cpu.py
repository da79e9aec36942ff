"""The C ABI on the host: the library loads, exports every declared symbol, and
rejects bad arguments with a status and a message (no GPU needed)."""
import ctypes
import glob
import os
import re

import pytest

from sparse_attention_indexer_start_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        from sparse_attention_indexer_start_amd import build
        build.build()
    return binding.load()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("dsa_select_init", "dsa_candidate_mask", "dsa_block_scores", "dsa_topk",
                 "dsa_select_fused"):
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def _shape(**kw):
    base = dict(rows=4, block_size=8, k_blocks=64, k_tokens=256, width=4096,
                row_stride=4096, col_stride=1, starts_repeat=1, ends_repeat=1)
    base.update(kw)
    return binding.Shape(base["rows"], base["block_size"], base["k_blocks"],
                         base["k_tokens"], base["width"], base["row_stride"],
                         base["col_stride"], base["starts_repeat"], base["ends_repeat"])


def _init(lib, shape, device=0):
    h = ctypes.c_void_p()
    rc = lib.dsa_select_init(ctypes.byref(shape) if shape is not None else None, device,
                             ctypes.byref(h))
    return rc, h


@pytest.mark.parametrize("kw,code", [
    (dict(block_size=0), -1),
    (dict(k_blocks=0), -1),
    (dict(k_tokens=0), -1),
    (dict(col_stride=0), -1),
    (dict(row_stride=0), -1),
    (dict(starts_repeat=0), -1),
    (dict(ends_repeat=0), -1),
    (dict(rows=-1), -1),
    (dict(width=-5), -1),
    (dict(width=1 << 31, row_stride=1 << 31), -2),
    (dict(row_stride=100), -1),                       # rows would overlap
    (dict(col_stride=2, row_stride=4096), -1),        # strided rows would overlap
    (dict(k_blocks=100000, k_tokens=100000), -2),
])
def test_init_rejects_bad_shapes(lib, kw, code):
    rc, h = _init(lib, _shape(**kw))
    assert rc == code
    assert not h.value
    assert lib.dsa_last_error().decode()


def test_init_rejects_null_and_negative_device(lib):
    rc, _ = _init(lib, None)
    assert rc == -1
    rc, _ = _init(lib, _shape(), device=-1)
    assert rc == -1
    assert lib.dsa_select_init(ctypes.byref(_shape()), 0, None) == -1


def test_calls_on_null_context_fail_cleanly(lib):
    assert lib.dsa_select_destroy(None) == -1
    assert lib.dsa_block_scores(None, None, None, None, None, None) == -1
    assert lib.dsa_topk(None, 0, None, None, None, None, None, None) == -1
    assert lib.dsa_candidate_mask(None, None, None, None, None, None) == -1
    assert lib.dsa_select_fused(None, None, None, None, None, None, None, 1, None) == -1
    v = ctypes.c_uint32()
    assert lib.dsa_read_status(None, ctypes.byref(v)) == -1
    assert lib.dsa_reset_workspace(None, None) == -1
    assert b"null context" in lib.dsa_last_error()


def test_valid_shape_without_device_reports_hip_error(lib):
    """Here there is no GPU: a valid shape gets as far as the HIP runtime and
    comes back as DSA_ERR_HIP.  On a GPU host it succeeds and is destroyed."""
    rc, h = _init(lib, _shape())
    if rc == 0:
        assert lib.dsa_select_destroy(h) == 0
    else:
        assert rc == -4
        assert lib.dsa_last_error().decode()
