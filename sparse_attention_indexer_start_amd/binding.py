"""ctypes binding of ``libdsa_select.so`` (argument marshalling only).

Every step of the selection runs in the HIP library; this module checks
tensor shapes, dtypes and devices on the host, passes raw device pointers and
the current HIP stream, and turns a negative status into an exception.  If the
library has not been built the first call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdsa_select.so")

DSA_TOPK_BLOCKS = 0
DSA_TOPK_TOKENS = 1
DSA_WRITE_MASK = 1
DSA_TWO_LAUNCHES = 2

STATUS_NAMES = {
    0: "DSA_OK", -1: "DSA_ERR_INVALID_ARG", -2: "DSA_ERR_UNSUPPORTED",
    -3: "DSA_ERR_CAPTURING", -4: "DSA_ERR_HIP", -5: "DSA_ERR_DESTROYED",
}

# Every entry point that include/dsa_select.h declares.
EXPORTED = (
    "dsa_select_init", "dsa_select_destroy", "dsa_select_query", "dsa_select_plan",
    "dsa_block_scores",
    "dsa_topk", "dsa_candidate_mask", "dsa_select_fused", "dsa_read_status",
    "dsa_reset_workspace", "dsa_last_error", "dsa_select_fused_noalloc",
    "dsa_indexer_select", "dsa_indexer_last_error",
    "dsa_row_topk_init", "dsa_row_topk_plan", "dsa_row_topk_destroy", "dsa_row_topk_pieces",
    "dsa_row_topk",
    "dsa_row_topk_last_error",
    "dsa_sparse_attn_init", "dsa_sparse_attn_plan", "dsa_sparse_attn_destroy",
    "dsa_sparse_attn_chunks",
    "dsa_sparse_attn", "dsa_sparse_attn_fp8", "dsa_sparse_attn_read_status",
    "dsa_sparse_attn_reset_status",
    "dsa_sparse_attn_last_error",
)


class DsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("k_blocks", ctypes.c_int32), ("k_tokens", ctypes.c_int32),
        ("width", ctypes.c_int64), ("row_stride", ctypes.c_int64),
        ("col_stride", ctypes.c_int64), ("starts_repeat", ctypes.c_int32),
        ("ends_repeat", ctypes.c_int32),
    ]


class LaunchInfo(ctypes.Structure):
    _fields_ = [
        ("programs_per_row", ctypes.c_int32), ("threads_per_group", ctypes.c_int32),
        ("grid_groups", ctypes.c_int32), ("small_row_blocks", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64), ("fused_launches", ctypes.c_int32),
    ]


class IndexerShape(ctypes.Structure):
    _fields_ = [
        ("queries", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("k_blocks", ctypes.c_int32), ("k_tokens", ctypes.c_int32),
        ("keys", ctypes.c_int64), ("starts_repeat", ctypes.c_int32),
        ("ends_repeat", ctypes.c_int32),
    ]


class TopkShape(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("k", ctypes.c_int32), ("width", ctypes.c_int64),
        ("row_stride", ctypes.c_int64), ("col_stride", ctypes.c_int64),
        ("starts_repeat", ctypes.c_int32), ("ends_repeat", ctypes.c_int32),
    ]


class AttnShape(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("group", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("k_tokens", ctypes.c_int32),
        ("rows_per_seq", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32), ("num_slots", ctypes.c_int64),
        ("k_slot_stride", ctypes.c_int64), ("k_head_stride", ctypes.c_int64),
        ("v_slot_stride", ctypes.c_int64), ("v_head_stride", ctypes.c_int64),
        ("chunks", ctypes.c_int32), ("union_rows", ctypes.c_int32),
    ]


class AttnPlanInfo(ctypes.Structure):
    _fields_ = [
        ("head_tiles", ctypes.c_int32), ("heads_per_tile", ctypes.c_int32),
        ("tiles_per_group", ctypes.c_int32), ("chunks", ctypes.c_int32),
        ("grid_groups", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64),
    ]


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return LIB_PATH


def load() -> ctypes.CDLL:
    """Load the library once; raise if it is not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_attention_indexer_start_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32
        lib.dsa_select_init.argtypes = [ctypes.POINTER(Shape), i32, ctypes.POINTER(vp)]
        lib.dsa_select_destroy.argtypes = [vp]
        lib.dsa_select_query.argtypes = [vp, ctypes.POINTER(LaunchInfo)]
        lib.dsa_select_plan.argtypes = [ctypes.POINTER(Shape), i32, ctypes.POINTER(LaunchInfo)]
        lib.dsa_block_scores.argtypes = [vp, vp, vp, vp, vp, vp]
        lib.dsa_topk.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp]
        lib.dsa_candidate_mask.argtypes = [vp, vp, vp, vp, vp, vp]
        lib.dsa_select_fused.argtypes = [vp, vp, vp, vp, vp, vp, vp, u32, vp]
        lib.dsa_read_status.argtypes = [vp, ctypes.POINTER(u32)]
        lib.dsa_reset_workspace.argtypes = [vp, vp]
        lib.dsa_select_fused_noalloc.argtypes = [ctypes.POINTER(Shape), i32, vp, vp, vp, vp,
                                                 vp, vp, u32, vp, vp]
        lib.dsa_indexer_select.argtypes = [ctypes.POINTER(IndexerShape), i32, vp, vp, vp, vp,
                                           vp, vp, vp, vp, vp, vp]
        lib.dsa_indexer_last_error.restype = ctypes.c_char_p
        lib.dsa_row_topk_init.argtypes = [ctypes.POINTER(TopkShape), i32, ctypes.POINTER(vp)]
        lib.dsa_row_topk_destroy.argtypes = [vp]
        lib.dsa_row_topk_pieces.argtypes = [vp]
        lib.dsa_row_topk_plan.argtypes = [ctypes.POINTER(TopkShape), i32,
                                          ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int64)]
        lib.dsa_row_topk.argtypes = [vp, vp, vp, vp, vp, vp]
        lib.dsa_row_topk_last_error.restype = ctypes.c_char_p
        lib.dsa_sparse_attn_init.argtypes = [ctypes.POINTER(AttnShape), i32, ctypes.POINTER(vp)]
        lib.dsa_sparse_attn_plan.argtypes = [ctypes.POINTER(AttnShape), i32,
                                             ctypes.POINTER(AttnPlanInfo)]
        lib.dsa_sparse_attn_destroy.argtypes = [vp]
        lib.dsa_sparse_attn_chunks.argtypes = [vp]
        lib.dsa_sparse_attn.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp]
        f32 = ctypes.c_float
        lib.dsa_sparse_attn_fp8.argtypes = [vp, vp, vp, vp, f32, f32, vp, vp, vp, f32, vp, vp, vp]
        lib.dsa_sparse_attn_read_status.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32)]
        lib.dsa_sparse_attn_reset_status.argtypes = [vp]
        lib.dsa_sparse_attn_last_error.restype = ctypes.c_char_p
        lib.dsa_last_error.restype = ctypes.c_char_p
        for name in EXPORTED:
            if not name.endswith("last_error"):
                getattr(lib, name).restype = i32
        _lib = lib
        return lib


def _check(rc: int) -> None:
    if rc != 0:
        msg = load().dsa_last_error().decode(errors="replace")
        raise DsaError(rc, msg)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def plan(rows: int, width: int, block_size: int, k_blocks: int, k_tokens: int, cus: int,
         row_stride: Optional[int] = None, col_stride: int = 1, starts_repeat: int = 1,
         ends_repeat: int = 1) -> LaunchInfo:
    """Launch geometry and workspace size of a shape on a device with ``cus``
    compute units (dsa_select_plan: host only, no device needed)."""
    shape = Shape(rows, block_size, k_blocks, k_tokens, width,
                  max(1, width * col_stride) if row_stride is None else row_stride,
                  col_stride, starts_repeat, ends_repeat)
    li = LaunchInfo()
    _check(load().dsa_select_plan(ctypes.byref(shape), cus, ctypes.byref(li)))
    return li


class Context:
    """One selection shape on one device (owns the library workspace).

    ``logits`` tensors passed to the methods must be fp32 views of shape
    ``[rows, width]`` with the strides given here (in elements); ``starts``
    (optional) and ``ends`` are int32, indexed by ``row // starts_repeat`` and
    ``row // ends_repeat``.
    """

    def __init__(self, rows: int, width: int, block_size: int, k_blocks: int,
                 k_tokens: int, row_stride: Optional[int] = None, col_stride: int = 1,
                 starts_repeat: int = 1, ends_repeat: int = 1, device: int = 0):
        lib = load()
        self.shape = Shape(rows, block_size, k_blocks, k_tokens, width,
                           max(1, width * col_stride) if row_stride is None else row_stride,
                           col_stride, starts_repeat, ends_repeat)
        self.device = device
        self.nblocks = -(-width // block_size) if width else 0
        h = ctypes.c_void_p()
        _check(lib.dsa_select_init(ctypes.byref(self.shape), device, ctypes.byref(h)))
        self._h = h

    # -- helpers ----------------------------------------------------------
    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            _check(load().dsa_select_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    @property
    def handle(self):
        if self._h is None:
            raise DsaError(-5, "context was closed")
        return self._h

    def info(self) -> LaunchInfo:
        li = LaunchInfo()
        _check(load().dsa_select_query(self.handle, ctypes.byref(li)))
        return li

    def _stream(self, stream):
        import torch
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        return ctypes.c_void_p(stream.cuda_stream)

    def _check_logits(self, t):
        import torch
        sh = self.shape
        if t.dtype != torch.float32 or not t.is_cuda:
            raise ValueError("logits must be a float32 device tensor")
        if tuple(t.shape) != (sh.rows, sh.width):
            raise ValueError(f"logits shape {tuple(t.shape)} != {(sh.rows, sh.width)}")
        if sh.rows and sh.width and (
                (sh.rows > 1 and t.stride(0) != sh.row_stride) or
                (sh.width > 1 and t.stride(1) != sh.col_stride)):
            raise ValueError(f"logits strides {t.stride()} != {(sh.row_stride, sh.col_stride)}")

    def _check_i32(self, t, name, n=None, shape=None):
        import torch
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
        if n is not None and t.numel() < n:
            raise ValueError(f"{name} has {t.numel()} elements, needs {n}")
        if shape is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != {shape}")

    def _check_bounds(self, starts, ends):
        sh = self.shape
        if starts is not None:
            self._check_i32(starts, "starts", -(-sh.rows // sh.starts_repeat))
        self._check_i32(ends, "ends", -(-sh.rows // sh.ends_repeat))

    # -- entry points -----------------------------------------------------
    def block_scores(self, logits, starts, ends, scores, stream=None):
        import torch
        self._check_logits(logits)
        self._check_bounds(starts, ends)
        if scores.dtype != torch.float32 or not scores.is_contiguous() or \
                tuple(scores.shape) != (self.shape.rows, self.nblocks):
            raise ValueError("scores must be contiguous float32 [rows, nblocks]")
        _check(load().dsa_block_scores(self.handle, _ptr(logits), _ptr(starts), _ptr(ends),
                                       _ptr(scores), self._stream(stream)))

    def topk_blocks(self, scores, starts, ends, out, stream=None):
        import torch
        self._check_bounds(starts, ends)
        if scores.dtype != torch.float32 or not scores.is_contiguous() or \
                tuple(scores.shape) != (self.shape.rows, self.nblocks):
            raise ValueError("scores must be contiguous float32 [rows, nblocks]")
        self._check_i32(out, "out", shape=(self.shape.rows, self.shape.k_blocks))
        _check(load().dsa_topk(self.handle, DSA_TOPK_BLOCKS, _ptr(scores), _ptr(starts),
                               _ptr(ends), None, _ptr(out), self._stream(stream)))

    def topk_tokens(self, logits, starts, ends, block_ids, out, stream=None):
        self._check_logits(logits)
        self._check_bounds(starts, ends)
        if block_ids is not None:
            self._check_i32(block_ids, "block_ids", shape=(self.shape.rows, self.shape.k_blocks))
        self._check_i32(out, "out", shape=(self.shape.rows, self.shape.k_tokens))
        _check(load().dsa_topk(self.handle, DSA_TOPK_TOKENS, _ptr(logits), _ptr(starts),
                               _ptr(ends), _ptr(block_ids), _ptr(out), self._stream(stream)))

    def candidate_mask(self, logits, starts, ends, block_ids, stream=None):
        self._check_logits(logits)
        self._check_bounds(starts, ends)
        self._check_i32(block_ids, "block_ids", shape=(self.shape.rows, self.shape.k_blocks))
        _check(load().dsa_candidate_mask(self.handle, _ptr(logits), _ptr(starts), _ptr(ends),
                                         _ptr(block_ids), self._stream(stream)))

    def select_fused(self, logits, starts, ends, block_ids, token_ids, scores=None,
                     write_mask: bool = True, stream=None, two_launches: bool = False):
        import torch
        self._check_logits(logits)
        self._check_bounds(starts, ends)
        self._check_i32(block_ids, "block_ids", shape=(self.shape.rows, self.shape.k_blocks))
        self._check_i32(token_ids, "token_ids", shape=(self.shape.rows, self.shape.k_tokens))
        if scores is not None and (scores.dtype != torch.float32 or not scores.is_contiguous()
                                   or tuple(scores.shape) != (self.shape.rows, self.nblocks)):
            raise ValueError("scores must be contiguous float32 [rows, nblocks]")
        _check(load().dsa_select_fused(self.handle, _ptr(logits), _ptr(starts), _ptr(ends),
                                       _ptr(block_ids), _ptr(token_ids), _ptr(scores),
                                       (DSA_WRITE_MASK if write_mask else 0)
                                       | (DSA_TWO_LAUNCHES if two_launches else 0),
                                       self._stream(stream)))

    def read_status(self) -> int:
        v = ctypes.c_uint32(0)
        _check(load().dsa_read_status(self.handle, ctypes.byref(v)))
        return v.value

    def reset_workspace(self, stream=None) -> None:
        _check(load().dsa_reset_workspace(self.handle, self._stream(stream)))


def select(logits, starts, ends, block_size: int, k_blocks: int, k_tokens: int,
           starts_repeat: int = 1, ends_repeat: int = 1, write_mask: bool = True,
           return_scores: bool = False):
    """One-shot fused selection; allocates the outputs with torch."""
    import torch
    rows, width = logits.shape
    ctx = Context(rows, width, block_size, k_blocks, k_tokens, row_stride=logits.stride(0),
                  col_stride=logits.stride(1), starts_repeat=starts_repeat,
                  ends_repeat=ends_repeat, device=logits.device.index or 0)
    bids = torch.empty((rows, k_blocks), dtype=torch.int32, device=logits.device)
    tids = torch.empty((rows, k_tokens), dtype=torch.int32, device=logits.device)
    sc = None
    if return_scores:
        sc = torch.full((rows, ctx.nblocks), float("-inf"), dtype=torch.float32, device=logits.device)
    ctx.select_fused(logits, starts, ends, bids, tids, sc, write_mask)
    torch.cuda.current_stream(logits.device).synchronize()
    ctx.close()
    return (bids, tids, sc) if return_scores else (bids, tids)


def select_fused_noalloc(logits, starts, ends, block_ids, token_ids, block_size: int,
                         k_blocks: int, k_tokens: int, scores=None, write_mask: bool = True,
                         starts_repeat: int = 1, ends_repeat: int = 1, status=None,
                         two_launches: bool = False, stream=None) -> None:
    """The allocation-free fused call (no context): the library's per-device
    scratch array is its workspace.  ``status`` is an optional int32 device
    tensor of one element, zeroed by the caller, into which status bits are
    ORed."""
    import torch
    rows, width = logits.shape
    if logits.dtype != torch.float32 or not logits.is_cuda:
        raise ValueError("logits must be a float32 device tensor")
    for t, name, shp in ((block_ids, "block_ids", (rows, k_blocks)),
                         (token_ids, "token_ids", (rows, k_tokens))):
        if t.dtype != torch.int32 or not t.is_contiguous() or tuple(t.shape) != shp:
            raise ValueError(f"{name} must be contiguous int32 {shp}")
    for t, name in ((starts, "starts"), (ends, "ends"), (status, "status")):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    nblocks = -(-width // block_size) if width else 0
    if scores is not None and (scores.dtype != torch.float32 or not scores.is_contiguous()
                               or tuple(scores.shape) != (rows, nblocks)):
        raise ValueError("scores must be contiguous float32 [rows, nblocks]")
    col_stride = logits.stride(1) if width > 1 else 1
    row_stride = logits.stride(0) if rows > 1 else max(1, width * col_stride)
    shape = Shape(rows, block_size, k_blocks, k_tokens, width, row_stride, col_stride,
                  starts_repeat, ends_repeat)
    dev = logits.device.index or 0
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    flags = (DSA_WRITE_MASK if write_mask else 0) | (DSA_TWO_LAUNCHES if two_launches else 0)
    _check(load().dsa_select_fused_noalloc(ctypes.byref(shape), dev, _ptr(logits), _ptr(starts),
                                           _ptr(ends), _ptr(block_ids), _ptr(token_ids),
                                           _ptr(scores), flags, _ptr(status),
                                           ctypes.c_void_p(stream.cuda_stream)))


def indexer_select(q8, k8, w, kscale, starts, ends, block_size: int, k_blocks: int,
                   k_tokens: int, starts_repeat: int = 1, ends_repeat: int = 1,
                   block_ids=None, token_ids=None, logits_out=None, stream=None):
    """The fused FP8 indexer logits plus selection (include/dsa_indexer.h).

    q8 uint8 [Q, H, D] and k8 uint8 [S, D] device tensors of E4M3 codes, w
    float32 [Q, H], kscale float32 [S] or None, starts/ends int32.  Returns
    (block_ids [Q, k_blocks], token_ids [Q, k_tokens]), allocated with torch
    when not given.  ``logits_out`` (float32 [Q, S]) receives the live logits.
    """
    import torch
    Q, H, D = q8.shape
    S = k8.shape[0]
    dev = q8.device
    for t, name, dt in ((q8, "q8", torch.uint8), (k8, "k8", torch.uint8),
                        (w, "w", torch.float32), (kscale, "kscale", torch.float32),
                        (starts, "starts", torch.int32), (ends, "ends", torch.int32),
                        (logits_out, "logits_out", torch.float32)):
        if t is not None and (t.dtype != dt or not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {dt} device tensor")
    if k8.dim() != 2 or k8.shape[1] != D or tuple(w.shape) != (Q, H):
        raise ValueError("k8 must be [S, D] and w [Q, H]")
    if kscale is not None and tuple(kscale.shape) != (S,):
        raise ValueError("kscale must be [S]")
    if ends is None or ends.numel() < -(-Q // ends_repeat):
        raise ValueError(f"ends needs {-(-Q // ends_repeat)} entries")
    if starts is not None and starts.numel() < -(-Q // starts_repeat):
        raise ValueError(f"starts needs {-(-Q // starts_repeat)} entries")
    if logits_out is not None and tuple(logits_out.shape) != (Q, S):
        raise ValueError("logits_out must be [Q, S]")
    if block_ids is None:
        block_ids = torch.empty((Q, k_blocks), dtype=torch.int32, device=dev)
    if token_ids is None:
        token_ids = torch.empty((Q, k_tokens), dtype=torch.int32, device=dev)
    for t, name, shp in ((block_ids, "block_ids", (Q, k_blocks)),
                         (token_ids, "token_ids", (Q, k_tokens))):
        if t.dtype != torch.int32 or not t.is_contiguous() or tuple(t.shape) != shp:
            raise ValueError(f"{name} must be contiguous int32 {shp}")
    shape = IndexerShape(Q, H, D, block_size, k_blocks, k_tokens, S, starts_repeat, ends_repeat)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    rc = load().dsa_indexer_select(ctypes.byref(shape), dev.index or 0, _ptr(q8), _ptr(k8),
                                   _ptr(w), _ptr(kscale), _ptr(starts), _ptr(ends),
                                   _ptr(block_ids), _ptr(token_ids), _ptr(logits_out),
                                   ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise DsaError(rc, load().dsa_indexer_last_error().decode(errors="replace"))
    return block_ids, token_ids


def row_topk_plan(rows: int, width: int, k: int, cus: int, col_stride: int = 1):
    """(pieces per row, workspace bytes) of a row top-k shape on a device with
    ``cus`` compute units (dsa_row_topk_plan: host only)."""
    shape = TopkShape(rows, k, width, max(1, width * col_stride), col_stride, 1, 1)
    p, w = ctypes.c_int32(), ctypes.c_int64()
    rc = load().dsa_row_topk_plan(ctypes.byref(shape), cus, ctypes.byref(p), ctypes.byref(w))
    if rc != 0:
        raise DsaError(rc, load().dsa_row_topk_last_error().decode(errors="replace"))
    return p.value, w.value


class RowTopk:
    """Cooperative per-row top-k for very long rows (include/dsa_row_topk.h)."""

    def __init__(self, rows: int, width: int, k: int, row_stride: Optional[int] = None,
                 col_stride: int = 1, starts_repeat: int = 1, ends_repeat: int = 1,
                 device: int = 0):
        lib = load()
        self.shape = TopkShape(rows, k, width,
                               max(1, width * col_stride) if row_stride is None else row_stride,
                               col_stride, starts_repeat, ends_repeat)
        self.device = device
        h = ctypes.c_void_p()
        self._check(lib.dsa_row_topk_init(ctypes.byref(self.shape), device, ctypes.byref(h)))
        self._h = h

    @staticmethod
    def _check(rc: int) -> None:
        if rc != 0:
            raise DsaError(rc, load().dsa_row_topk_last_error().decode(errors="replace"))

    def pieces(self) -> int:
        n = load().dsa_row_topk_pieces(self._h)
        if n < 0:
            self._check(n)
        return n

    def __call__(self, logits, starts, ends, out=None, stream=None):
        import torch
        sh = self.shape
        if logits.dtype != torch.float32 or not logits.is_cuda:
            raise ValueError("logits must be a float32 device tensor")
        if tuple(logits.shape) != (sh.rows, sh.width):
            raise ValueError(f"logits shape {tuple(logits.shape)} != {(sh.rows, sh.width)}")
        if sh.rows > 1 and sh.width > 0 and logits.stride(0) != sh.row_stride:
            raise ValueError("logits row stride differs from the context's")
        if sh.width > 1 and logits.stride(1) != sh.col_stride:
            raise ValueError("logits column stride differs from the context's")
        for t, name, n in ((starts, "starts", -(-sh.rows // sh.starts_repeat)),
                           (ends, "ends", -(-sh.rows // sh.ends_repeat))):
            if t is None:
                if name == "ends":
                    raise ValueError("ends is required")
                continue
            if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() < n:
                raise ValueError(f"{name} must be a contiguous int32 tensor of >= {n} entries")
        if out is None:
            out = torch.empty((sh.rows, sh.k), dtype=torch.int32, device=logits.device)
        if out.dtype != torch.int32 or not out.is_contiguous() or tuple(out.shape) != (sh.rows, sh.k):
            raise ValueError(f"out must be contiguous int32 {(sh.rows, sh.k)}")
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        self._check(load().dsa_row_topk(self._h, _ptr(logits), _ptr(starts), _ptr(ends),
                                        _ptr(out), ctypes.c_void_p(stream.cuda_stream)))
        return out

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._check(load().dsa_row_topk_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def attn_plan(rows: int, kv_heads: int, group: int, head_dim: int, k_tokens: int, cus: int,
              num_slots: int = 1, rows_per_seq: int = 1, chunks: int = 0,
              union_rows: int = 0) -> AttnPlanInfo:
    """Launch plan of a sparse-attention shape on a device with ``cus`` compute
    units (dsa_sparse_attn_plan: host only, contiguous caches assumed)."""
    shape = AttnShape(rows, kv_heads, group, head_dim, k_tokens, rows_per_seq, 1, 0, num_slots,
                      kv_heads * head_dim, head_dim, kv_heads * head_dim, head_dim, chunks,
                      union_rows)
    li = AttnPlanInfo()
    rc = load().dsa_sparse_attn_plan(ctypes.byref(shape), cus, ctypes.byref(li))
    if rc != 0:
        raise DsaError(rc, load().dsa_sparse_attn_last_error().decode(errors="replace"))
    return li


class SparseAttn:
    """Sparse attention over each row's selected tokens (include/dsa_sparse_attn.h).

    The caches are bf16 tensors [num_slots, kv_heads, head_dim], or uint8
    tensors of E4M3 codes with k_scale and v_scale given (any slot and head
    strides that are multiples of 8 elements, innermost dimension
    contiguous); q and gate are bf16 [rows, kv_heads * group, head_dim].
    union_rows >= 2 selects union mode: each group of that many consecutive rows
    is attended in one pass over the union of its ids."""

    def __init__(self, rows: int, kv_heads: int, group: int, head_dim: int, k_tokens: int,
                 num_slots: int, rows_per_seq: int = 1, page_size: int = 1,
                 pages_per_seq: int = 0, k_strides=None, v_strides=None, chunks: int = 0,
                 device: int = 0, union_rows: int = 0):
        lib = load()
        ks = (kv_heads * head_dim, head_dim) if k_strides is None else tuple(k_strides)
        vs = (kv_heads * head_dim, head_dim) if v_strides is None else tuple(v_strides)
        self.shape = AttnShape(rows, kv_heads, group, head_dim, k_tokens, rows_per_seq,
                               page_size, pages_per_seq, num_slots, ks[0], ks[1], vs[0], vs[1],
                               chunks, union_rows)
        self.device = device
        h = ctypes.c_void_p()
        self._check(lib.dsa_sparse_attn_init(ctypes.byref(self.shape), device, ctypes.byref(h)))
        self._h = h

    @staticmethod
    def _check(rc: int) -> None:
        if rc != 0:
            raise DsaError(rc, load().dsa_sparse_attn_last_error().decode(errors="replace"))

    def chunks(self) -> int:
        n = load().dsa_sparse_attn_chunks(self._h)
        if n < 0:
            self._check(n)
        return n

    def read_status(self) -> int:
        v = ctypes.c_uint32(0)
        self._check(load().dsa_sparse_attn_read_status(self._h, ctypes.byref(v)))
        return v.value

    def reset_status(self) -> None:
        self._check(load().dsa_sparse_attn_reset_status(self._h))

    def __call__(self, q, k_cache, v_cache, token_ids, page_table=None, gate=None,
                 sm_scale=None, out=None, lse=None, stream=None, k_scale=None, v_scale=None):
        import torch
        sh = self.shape
        fp8 = k_cache.dtype == torch.uint8
        if fp8 != (v_cache.dtype == torch.uint8) or fp8 != (k_scale is not None) \
                or fp8 != (v_scale is not None):
            raise ValueError("fp8 caches are uint8 (both) and need k_scale and v_scale")
        hq = sh.kv_heads * sh.group
        D = sh.head_dim
        for t, name in ((q, "q"), (gate, "gate")):
            if t is None:
                continue
            if (t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous()
                    or tuple(t.shape) != (sh.rows, hq, D)):
                raise ValueError(f"{name} must be contiguous bf16 {(sh.rows, hq, D)}")
        for t, name, st in ((k_cache, "k_cache", (sh.k_slot_stride, sh.k_head_stride)),
                            (v_cache, "v_cache", (sh.v_slot_stride, sh.v_head_stride))):
            if t.dtype not in (torch.bfloat16, torch.uint8) or not t.is_cuda or t.dim() != 3:
                raise ValueError(f"{name} must be a 3-d bf16 or uint8 device tensor")
            if t.shape[0] < sh.num_slots or t.shape[1] != sh.kv_heads or t.shape[2] != D:
                raise ValueError(f"{name} shape {tuple(t.shape)} does not hold "
                                 f"{(sh.num_slots, sh.kv_heads, D)}")
            if t.stride(2) != 1 or (t.stride(0), t.stride(1)) != st:
                raise ValueError(f"{name} strides {t.stride()} differ from the context's {st}")
        if (token_ids.dtype != torch.int32 or not token_ids.is_contiguous()
                or tuple(token_ids.shape) != (sh.rows, sh.k_tokens)):
            raise ValueError(f"token_ids must be contiguous int32 {(sh.rows, sh.k_tokens)}")
        if page_table is not None:
            nseq = -(-sh.rows // sh.rows_per_seq)
            if (page_table.dtype != torch.int32 or not page_table.is_contiguous()
                    or page_table.dim() != 2 or page_table.shape[0] < nseq
                    or page_table.shape[1] != sh.pages_per_seq):
                raise ValueError(f"page_table must be contiguous int32 [>= {nseq}, "
                                 f"{sh.pages_per_seq}]")
        if sm_scale is None:
            sm_scale = 1.0 / (D ** 0.5)
        if out is None:
            out = torch.empty((sh.rows, hq, D), dtype=torch.bfloat16, device=q.device)
        if (out.dtype != torch.bfloat16 or not out.is_contiguous()
                or tuple(out.shape) != (sh.rows, hq, D)):
            raise ValueError(f"out must be contiguous bf16 {(sh.rows, hq, D)}")
        if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                                or tuple(lse.shape) != (sh.rows, hq)):
            raise ValueError(f"lse must be contiguous float32 {(sh.rows, hq)}")
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        if fp8:
            self._check(load().dsa_sparse_attn_fp8(
                self._h, _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.c_float(k_scale),
                ctypes.c_float(v_scale), _ptr(token_ids), _ptr(page_table), _ptr(gate),
                ctypes.c_float(sm_scale), _ptr(out), _ptr(lse),
                ctypes.c_void_p(stream.cuda_stream)))
        else:
            self._check(load().dsa_sparse_attn(
                self._h, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(token_ids),
                _ptr(page_table), _ptr(gate), ctypes.c_float(sm_scale), _ptr(out), _ptr(lse),
                ctypes.c_void_p(stream.cuda_stream)))
        return out

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._check(load().dsa_sparse_attn_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
