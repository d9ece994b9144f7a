"""ctypes binding of the C ABI declared in ``include/sparse_attn.h``.

Argument marshalling only: every step of the attention runs in the HIP
library.  PyTorch supplies device memory (``torch.empty``) and the current
stream.  The library is loaded on first use; if it has not been built the
call raises (there is no fallback).
"""

from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libsparse_attn.so"

# enum values of sparse_attn.h
SA_OK, SA_EINVAL, SA_EUNSUPPORTED, SA_ESIZE, SA_EHIP, SA_ENOMEM = 0, -1, -2, -3, -4, -5
KINDS = {"local": 0, "stride": 1, "sameblock": 2, "summary": 3, "fixed_merged": 4,
         "local_global": 5, "strided_merged": 6}
SA_STRIDE_FAR = 7  # blob-only pattern kind: second part of a merged strided head
PART_INIT = 1 << 30  # schedule pattern field: first chunk starts from the part state
SA_BF16, SA_FP32 = 0, 1
SA_SELF_IF_EMPTY = 1
SA_NO_SEGMENT_PASS = 2
SA_BLOB_MAGIC = 0x31415053
SA_TILE_PARTIAL, SA_TILE_FULL = 0, 1
SA_XCDS = 8

EXPORTED = (
    "sparse_attn_layout", "sparse_attn_layout_check", "sparse_attn_fwd_workspace",
    "sparse_attn_fwd", "sparse_attn_fwd_phases", "sparse_attn_bwd_workspace",
    "sparse_attn_bwd", "sparse_attn_bwd_phases", "sparse_attn_bwd_static", "sparse_attn_strerror",
)
SA_STATIC_SCRATCH_BYTES = 64 << 20  # sparse_attn.h: device array of sparse_attn_bwd_static
SA_FWD_MAIN, SA_FWD_MERGE, SA_FWD_ALL = 1, 2, 3
SA_BWD_DQ, SA_BWD_DKDV, SA_BWD_MERGE, SA_BWD_SEG, SA_BWD_ALL = 1, 2, 4, 8, 15
SA_SCHED_FIELDS = 9
SA_SEGMENT_ROWS = 128


class CHeadPattern(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("l", ctypes.c_int32), ("c", ctypes.c_int32),
                ("sub", ctypes.c_int32)]


class CLayoutDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("heads", ctypes.POINTER(CHeadPattern)),
                ("flags", ctypes.c_uint32), ("split_keys", ctypes.c_int32),
                ("split_rows", ctypes.c_int32)]


class CPatternRec(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("l", ctypes.c_int32), ("c", ctypes.c_int32),
                ("sub", ctypes.c_int32), ("s", ctypes.c_int32), ("nnz", ctypes.c_int32),
                ("pairs", ctypes.c_int64)] + [
        (f, ctypes.c_int64) for f in ("qmap_off", "kmap_off", "lo_off", "hi_off", "pre_off", "count_off",
                                      "row_ptr_off", "col_off", "fflag_off", "col_ptr_off",
                                      "row_off", "bflag_off")]


class CBlobHeader(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32), ("n", ctypes.c_int64),
                ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("num_patterns", ctypes.c_int32),
                ("n_pad", ctypes.c_int32), ("nqt", ctypes.c_int32), ("nkt", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("total_bytes", ctypes.c_int64),
                ("head_pattern_off", ctypes.c_int64), ("pattern_off", ctypes.c_int64),
                ("fwd_sched_off", ctypes.c_int64), ("bwd_sched_off", ctypes.c_int64),
                ("fwd_sched_len", ctypes.c_int32), ("bwd_sched_len", ctypes.c_int32),
                ("red_sched_off", ctypes.c_int64), ("red_sched_len", ctypes.c_int32),
                ("num_slots", ctypes.c_int32),
                ("fwd_xl_off", ctypes.c_int64), ("bwd_xl_off", ctypes.c_int64),
                ("fwd_xl_len", ctypes.c_int32), ("bwd_xl_len", ctypes.c_int32),
                ("fwd_xitem_off", ctypes.c_int64), ("bwd_xitem_off", ctypes.c_int64),
                ("comb_sched_off", ctypes.c_int64), ("comb_sched_len", ctypes.c_int32),
                ("num_qslots", ctypes.c_int32),
                ("split_keys", ctypes.c_int32), ("split_rows", ctypes.c_int32),
                ("pairs_all_heads", ctypes.c_int64), ("tiles_all_heads", ctypes.c_int64),
                ("head_part_off", ctypes.c_int64), ("head_merged_off", ctypes.c_int64),
                ("num_merged", ctypes.c_int32), ("fwdp_sched_len", ctypes.c_int32),
                ("bwdp_sched_len", ctypes.c_int32), ("fwdp_xl_len", ctypes.c_int32),
                ("bwdp_xl_len", ctypes.c_int32), ("pad0", ctypes.c_int32),
                ("fwdp_sched_off", ctypes.c_int64), ("bwdp_sched_off", ctypes.c_int64),
                ("fwdp_xitem_off", ctypes.c_int64), ("bwdp_xitem_off", ctypes.c_int64),
                ("dq_xl_len", ctypes.c_int32), ("seg_xl_len", ctypes.c_int32),
                ("seg_len", ctypes.c_int32), ("seg_tiles", ctypes.c_int32),
                ("dq_xitem_off", ctypes.c_int64), ("seg_xitem_off", ctypes.c_int64)]


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_strerror(status)} (status {status})")


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return os.path.join(_PKG, LIB_NAME)


def load_library():
    """Load the built library (raises RuntimeError if it is missing)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{LIB_NAME} is not built ({path}); run `python -m factorized_block_sparse_amd.build`")
        _lib = configure(ctypes.CDLL(path))
        return _lib


def configure(lib):
    """Declare the argument and result types of the C ABI on a loaded library."""
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.sparse_attn_layout.argtypes = [ctypes.POINTER(CLayoutDesc), vp, ctypes.POINTER(sz)]
    lib.sparse_attn_layout.restype = i32
    lib.sparse_attn_layout_check.argtypes = [vp, sz]
    lib.sparse_attn_layout_check.restype = i32
    lib.sparse_attn_fwd_workspace.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.sparse_attn_fwd_workspace.restype = i32
    lib.sparse_attn_fwd.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, f32, vp]
    lib.sparse_attn_fwd.restype = i32
    lib.sparse_attn_fwd_phases.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz,
                                           f32, ctypes.c_uint, vp]
    lib.sparse_attn_fwd_phases.restype = i32
    lib.sparse_attn_bwd_workspace.argtypes = [vp, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.sparse_attn_bwd_workspace.restype = i32
    lib.sparse_attn_bwd.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                    vp, vp, sz, f32, vp]
    lib.sparse_attn_bwd.restype = i32
    lib.sparse_attn_bwd_phases.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                           vp, vp, vp, sz, f32, ctypes.c_uint, vp]
    lib.sparse_attn_bwd_phases.restype = i32
    lib.sparse_attn_bwd_static.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                           vp, vp, vp, f32, vp]
    lib.sparse_attn_bwd_static.restype = i32
    lib.sparse_attn_strerror.argtypes = [i32]
    lib.sparse_attn_strerror.restype = ctypes.c_char_p
    return lib


def _strerror(status: int) -> str:
    try:
        return load_library().sparse_attn_strerror(status).decode()
    except RuntimeError:
        return "library not loaded"


def _check(rc: int, what: str):
    if rc != SA_OK:
        raise SparseAttnError(rc, what)


@dataclass(frozen=True)
class HeadPattern:
    """One head's pattern: kind in {"local", "stride", "sameblock", "summary",
    "fixed_merged", "local_global", "strided_merged"}; c is the summary width,
    or for "local_global" the number of leading global tokens."""
    kind: str
    l: int
    c: int = 0
    sub: int = 0

    def to_c(self) -> CHeadPattern:
        if self.kind not in KINDS:
            raise ValueError(f"unknown head kind {self.kind!r}")
        return CHeadPattern(KINDS[self.kind], self.l, self.c, self.sub)


def sparse_attn_layout(n: int, heads, block_q: int = 64, block_k: int = 64,
                       self_if_empty: bool = True, split_keys: int = 0,
                       split_rows: int = 0, segment_pass: bool = True) -> np.ndarray:
    """Build the layout blob (host bytes) for ``heads`` at sequence length ``n``.

    ``split_keys`` / ``split_rows`` are the chunk caps of the forward / dQ and
    dK/dV schedules (0 = the library defaults); ``segment_pass=False`` builds
    it with SA_NO_SEGMENT_PASS."""
    lib = load_library()
    heads = [h if isinstance(h, HeadPattern) else HeadPattern(h.kind, h.l, h.c, h.sub) for h in heads]
    arr = (CHeadPattern * max(1, len(heads)))(*[h.to_c() for h in heads])
    flags = (SA_SELF_IF_EMPTY if self_if_empty else 0) | (0 if segment_pass else SA_NO_SEGMENT_PASS)
    desc = CLayoutDesc(n, block_q, block_k, len(heads), arr, flags, split_keys, split_rows)
    size = ctypes.c_size_t(0)
    _check(lib.sparse_attn_layout(ctypes.byref(desc), None, ctypes.byref(size)), "layout size")
    blob = np.zeros(size.value, dtype=np.uint8)
    _check(lib.sparse_attn_layout(ctypes.byref(desc), blob.ctypes.data_as(ctypes.c_void_p),
                                  ctypes.byref(size)), "layout build")
    return blob[: size.value]


class Layout:
    """A built layout: the host blob plus lazily made device copies (one per device)."""

    def __init__(self, n: int, heads, block_q: int = 64, block_k: int = 64,
                 self_if_empty: bool = True, split_keys: int = 0, split_rows: int = 0,
                 segment_pass: bool = True):
        self.n = int(n)
        self.heads = tuple(heads)
        self.blob = sparse_attn_layout(n, heads, block_q, block_k, self_if_empty, split_keys,
                                       split_rows, segment_pass)
        self.header = CBlobHeader.from_buffer_copy(self.blob[: ctypes.sizeof(CBlobHeader)].tobytes())
        self._dev = {}

    # -- host-side views (tests, accounting) --------------------------------
    def _arr(self, off: int, count: int, dtype) -> np.ndarray:
        nbytes = count * np.dtype(dtype).itemsize
        return self.blob[off: off + nbytes].view(dtype)

    @property
    def num_patterns(self) -> int:
        return self.header.num_patterns

    def head_pattern_index(self) -> np.ndarray:
        return self._arr(self.header.head_pattern_off, self.header.num_heads, np.int32)

    def pattern_rec(self, i: int) -> CPatternRec:
        off = self.header.pattern_off + i * ctypes.sizeof(CPatternRec)
        return CPatternRec.from_buffer_copy(self.blob[off: off + ctypes.sizeof(CPatternRec)].tobytes())

    def pattern_arrays(self, i: int) -> dict:
        r, h = self.pattern_rec(i), self.header
        return {
            "qmap": self._arr(r.qmap_off, h.n_pad, np.int32),
            "kmap": self._arr(r.kmap_off, h.n_pad, np.int32),
            "lo": self._arr(r.lo_off, h.n_pad, np.int32),
            "hi": self._arr(r.hi_off, h.n_pad, np.int32),
            "pre": (self._arr(r.pre_off, h.n_pad, np.int32) if r.pre_off
                    else np.zeros(h.n_pad, dtype=np.int32)),
            "count": self._arr(r.count_off, h.n, np.int32),
            "row_ptr": self._arr(r.row_ptr_off, h.nqt + 1, np.int32),
            "col": self._arr(r.col_off, r.nnz, np.int32),
            "fflag": self._arr(r.fflag_off, r.nnz, np.uint8),
            "col_ptr": self._arr(r.col_ptr_off, h.nkt + 1, np.int32),
            "row": self._arr(r.row_off, r.nnz, np.int32),
            "bflag": self._arr(r.bflag_off, r.nnz, np.uint8),
        }

    def fwd_schedule(self) -> np.ndarray:
        """Rows (head, q-tile, first CSR entry, end CSR entry, partial slot, pattern index,
        first slot of the tile, chunks of the tile, first entry's tile as (tile << 1) | FULL
        or -1); slot = slot0 = -1, chunks = 1 for unsplit tiles."""
        return self._arr(self.header.fwd_sched_off, SA_SCHED_FIELDS * self.header.fwd_sched_len,
                         np.int32).reshape(-1, SA_SCHED_FIELDS)

    def combine_schedule(self) -> np.ndarray:
        """Rows (head, q-tile, first partial slot, chunks) of the split query tiles."""
        return self._arr(self.header.comb_sched_off, 4 * self.header.comb_sched_len, np.int32).reshape(-1, 4)

    def bwd_schedule(self) -> np.ndarray:
        """Rows as fwd_schedule over (head, k-tile) and CSC entries."""
        return self._arr(self.header.bwd_sched_off, SA_SCHED_FIELDS * self.header.bwd_sched_len,
                         np.int32).reshape(-1, SA_SCHED_FIELDS)

    def xcd_items(self, which: str) -> np.ndarray:
        """[SA_XCDS, len, SA_SCHED_FIELDS] schedule entries in list order ("fwd", "bwd",
        "fwdp" / "bwdp" for the second parts of two-part heads, "dq" for the dQ pass,
        "seg" for the segments of the segment pass)."""
        h = self.header
        off, ln = {"fwd": (h.fwd_xitem_off, h.fwd_xl_len), "bwd": (h.bwd_xitem_off, h.bwd_xl_len),
                   "fwdp": (h.fwdp_xitem_off, h.fwdp_xl_len),
                   "bwdp": (h.bwdp_xitem_off, h.bwdp_xl_len),
                   "dq": (h.dq_xitem_off, h.dq_xl_len), "seg": (h.seg_xitem_off, h.seg_xl_len)}[which]
        return self._arr(off, SA_XCDS * ln * SA_SCHED_FIELDS, np.int32).reshape(SA_XCDS, ln, SA_SCHED_FIELDS)

    def part_schedules(self) -> tuple:
        """(forward, backward) schedules of the second parts of two-part heads, rows as
        fwd_schedule (every tile holding a token, none split)."""
        h = self.header
        f = self._arr(h.fwdp_sched_off, SA_SCHED_FIELDS * h.fwdp_sched_len, np.int32)
        b = self._arr(h.bwdp_sched_off, SA_SCHED_FIELDS * h.bwdp_sched_len, np.int32)
        return f.reshape(-1, SA_SCHED_FIELDS), b.reshape(-1, SA_SCHED_FIELDS)

    def head_parts(self) -> tuple:
        """(second-part pattern index or -1, index among two-part heads or -1) per head."""
        h = self.header
        return (self._arr(h.head_part_off, h.num_heads, np.int32),
                self._arr(h.head_merged_off, h.num_heads, np.int32))

    def xcd_lists(self, which: str) -> np.ndarray:
        """[SA_XCDS, len] schedule indices per XCD ("fwd" or "bwd"), -1 = padding."""
        h = self.header
        off, ln = (h.fwd_xl_off, h.fwd_xl_len) if which == "fwd" else (h.bwd_xl_off, h.bwd_xl_len)
        return self._arr(off, SA_XCDS * ln, np.int32).reshape(SA_XCDS, ln)

    def reduce_schedule(self) -> np.ndarray:
        """Rows (head, k-tile, first partial slot, chunks) of the split key tiles."""
        return self._arr(self.header.red_sched_off, 4 * self.header.red_sched_len, np.int32).reshape(-1, 4)

    def pairs_per_batch(self) -> int:
        """Visible (query, key) pairs summed over the heads of one batch element."""
        return int(self.header.pairs_all_heads)

    def tiles_per_batch(self) -> int:
        return int(self.header.tiles_all_heads)

    # -- device copy ---------------------------------------------------------
    def device_blob(self, device):
        import torch
        dev = torch.device(device)
        key = (dev.type, dev.index)
        t = self._dev.get(key)
        if t is None:
            t = torch.from_numpy(self.blob.copy()).to(dev)
            self._dev[key] = t
        return t


def _ptr(t) -> int:
    return t.data_ptr()


def _check_qkv(layout: Layout, tensors, names):
    import torch
    ref = tensors[0]
    if ref.dim() != 4:
        raise ValueError("tensors must be [B, H, n, d]")
    for t, nm in zip(tensors, names):
        if not t.is_cuda:
            raise ValueError(f"{nm} must be a GPU tensor")
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError(f"{nm} must match q in shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    B, H, n, d = ref.shape
    if n != layout.n or H != layout.header.num_heads:
        raise ValueError(f"layout is for n={layout.n}, H={layout.header.num_heads}; got n={n}, H={H}")
    if ref.dtype == torch.bfloat16:
        dt = SA_BF16
    elif ref.dtype == torch.float32:
        dt = SA_FP32
    else:
        raise ValueError("dtype must be bfloat16 or float32")
    return B, H, n, d, dt


def _check_like(t, ref, nm):
    """An output tensor the kernels write through a raw pointer: same shape,
    dtype and device as ``ref``, contiguous."""
    if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device or not t.is_contiguous():
        raise ValueError(f"{nm} must be a contiguous tensor of q's shape, dtype and device")


def _check_lse(lse, B, H, n, device, nm="lse"):
    import torch
    if (tuple(lse.shape) != (B, H, n) or lse.dtype != torch.float32 or lse.device != device
            or not lse.is_contiguous()):
        raise ValueError(f"{nm} must be a contiguous float32 [B, H, n] tensor on q's device")


def _check_workspace(ws, device):
    import torch
    if ws.dtype != torch.uint8 or ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on q's device")


def fwd_workspace_bytes(layout: Layout, B: int, H: int, d: int = 64, dtype: int = SA_BF16) -> int:
    lib = load_library()
    size = ctypes.c_size_t(0)
    _check(lib.sparse_attn_fwd_workspace(layout.blob.ctypes.data, B, H, d, dtype,
                                         ctypes.byref(size)), "sparse_attn_fwd_workspace")
    return size.value


def sparse_attn_fwd(layout: Layout, q, k, v, scale: float | None = None, out=None, lse=None,
                    workspace=None, phases: int = SA_FWD_ALL):
    """Forward on the current torch stream: returns (o, lse).

    ``workspace``: a uint8 device tensor of at least ``fwd_workspace_bytes``
    bytes (allocated when omitted).  ``phases`` selects which of the two
    launches run (``sparse_attn_fwd_phases`` in the C header).
    """
    import torch
    lib = load_library()
    B, H, n, d, dt = _check_qkv(layout, (q, k, v), ("q", "k", "v"))
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, H, n), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_like(o, q, "out")
    _check_lse(lse_t, B, H, n, q.device)
    if workspace is not None:
        _check_workspace(workspace, q.device)
    if workspace is None:
        need = fwd_workspace_bytes(layout, B, H, d, dt)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    ws_ptr = 0 if workspace is None else _ptr(workspace)
    ws_len = 0 if workspace is None else workspace.numel()
    blob_dev = layout.device_blob(q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    args = (layout.blob.ctypes.data, _ptr(blob_dev), B, H, d, dt, _ptr(q), _ptr(k), _ptr(v),
            _ptr(o), _ptr(lse_t), ws_ptr, ws_len, 0.0 if scale is None else float(scale))
    if phases == SA_FWD_ALL:
        rc = lib.sparse_attn_fwd(*args, stream)
    else:
        rc = lib.sparse_attn_fwd_phases(*args, phases, stream)
    _check(rc, "sparse_attn_fwd")
    return o, lse_t


def bwd_workspace_bytes(layout: Layout, B: int, H: int, d: int = 64, dtype: int = SA_BF16) -> int:
    lib = load_library()
    size = ctypes.c_size_t(0)
    _check(lib.sparse_attn_bwd_workspace(layout.blob.ctypes.data, B, H, d, dtype,
                                         ctypes.byref(size)), "sparse_attn_bwd_workspace")
    return size.value


def sparse_attn_bwd(layout: Layout, q, k, v, o, lse, do, scale: float | None = None,
                    workspace=None, grads=None, phases: int = SA_BWD_ALL):
    """Backward on the current torch stream: returns (dq, dk, dv).

    ``phases`` selects which of the backward's launches run (see
    ``sparse_attn_bwd_phases`` in the C header); the default runs all.
    ``workspace``: a uint8 device tensor of at least ``bwd_workspace_bytes``
    bytes (allocated when omitted).
    """
    import torch
    lib = load_library()
    B, H, n, d, dt = _check_qkv(layout, (q, k, v, o, do), ("q", "k", "v", "o", "do"))
    _check_lse(lse, B, H, n, q.device)
    need = bwd_workspace_bytes(layout, B, H, d, dt)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    _check_workspace(ws, q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_like(t, q, nm)
    blob_dev = layout.device_blob(q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    args = (layout.blob.ctypes.data, _ptr(blob_dev), B, H, d, dt,
            _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(),
            0.0 if scale is None else float(scale))
    if phases == SA_BWD_ALL:
        rc = lib.sparse_attn_bwd(*args, stream)
    else:
        rc = lib.sparse_attn_bwd_phases(*args, phases, stream)
    _check(rc, "sparse_attn_bwd")
    return dq, dk, dv


def sparse_attn_bwd_static(layout: Layout, q, k, v, o, lse, do, scale: float | None = None,
                           grads=None):
    """Backward through the allocation-free entry point (``sparse_attn_bwd_static``):
    the library's own per-GPU device array serves as workspace.  Returns
    (dq, dk, dv); pass ``grads`` to write into existing tensors (then nothing
    is allocated by this call either).  Calls on one GPU must not overlap."""
    import torch
    lib = load_library()
    B, H, n, d, dt = _check_qkv(layout, (q, k, v, o, do), ("q", "k", "v", "o", "do"))
    _check_lse(lse, B, H, n, q.device)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_like(t, q, nm)
    blob_dev = layout.device_blob(q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = lib.sparse_attn_bwd_static(layout.blob.ctypes.data, _ptr(blob_dev), B, H, d, dt,
                                    _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                    _ptr(dq), _ptr(dk), _ptr(dv),
                                    0.0 if scale is None else float(scale), stream)
    if rc == SA_ESIZE:
        need = bwd_workspace_bytes(layout, B, H, d, dt)
        raise SparseAttnError(rc, f"sparse_attn_bwd_static: these sizes need {need} bytes of "
                                  f"workspace, the static array holds {SA_STATIC_SCRATCH_BYTES}")
    _check(rc, "sparse_attn_bwd_static")
    return dq, dk, dv
