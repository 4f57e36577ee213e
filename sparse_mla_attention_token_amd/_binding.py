"""ctypes binding of the C ABI in include/smla.h (argument marshalling only).

Every step of the attention runs in the HIP kernels of libsmla.so; this
module only turns torch tensors into device pointers and sizes.  There is no
CPU fallback: if the library is missing or a call fails, an exception is
raised.
"""

from __future__ import annotations

import ctypes
import os
from pathlib import Path
from typing import Optional

import torch

_PKG = Path(__file__).resolve().parent
LIB_PATH = Path(os.environ.get("SMLA_LIB", _PKG / "libsmla.so"))

QK_DEPTH = 576
V_DEPTH = 512

SMLA_OK = 0
STATUS_NAMES = {
    0: "SMLA_OK",
    1: "SMLA_ERR_NULL",
    2: "SMLA_ERR_SHAPE",
    3: "SMLA_ERR_UNSUPPORTED",
    4: "SMLA_ERR_MISALIGNED",
    5: "SMLA_ERR_LAUNCH",
    6: "SMLA_ERR_SCRATCH_LIMIT",
}

EXPORTED_SYMBOLS = ("sparse_mla_prefill", "sparse_mla_prefill_split", "sparse_mla_prefill_single_pass",
                    "sparse_mla_prefill_split_noalloc", "sparse_mla_noalloc_scratch_bytes",
                    "sparse_mla_split_workspace_bytes", "sparse_mla_auto_splits", "sparse_mla_gather_debug",
                    "sparse_mla_index_scores", "sparse_mla_index_topk", "mla_dense_prefill", "smla_status_string",
                    "smla_version")

INDEX_DEPTH = 128


class SmlaDims(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("qk_depth", ctypes.c_int32),
        ("v_depth", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
    ]


class SmlaIndexDims(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("depth", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("score_stride", ctypes.c_int32),
        ("topk", ctypes.c_int32),
    ]


class SmlaDenseDims(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("max_prompt_len", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("nope_depth", ctypes.c_int32),
        ("rope_depth", ctypes.c_int32),
        ("v_depth", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("causal", ctypes.c_int32),
    ]


class SmlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {STATUS_NAMES.get(status, status)}")


_lib = None


def load_library(path: Optional[Path] = None) -> ctypes.CDLL:
    """Load libsmla.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise ImportError(f"{p} not found: build it with __graft_entry__.build() "
                          "or python sparse_mla_attention_token_amd/build.py")
    lib = ctypes.CDLL(str(p))
    vp, i32p, u32p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    lib.sparse_mla_prefill.restype = ctypes.c_int
    lib.sparse_mla_prefill.argtypes = [vp, vp, vp, i32p, i32p, f32p, u32p, u32p, f32p, ctypes.c_float,
                                       ctypes.c_int32, ctypes.POINTER(SmlaDims), vp]
    lib.sparse_mla_prefill_split.restype = ctypes.c_int
    lib.sparse_mla_prefill_split.argtypes = [vp, vp, vp, i32p, i32p, f32p, u32p, u32p, f32p, ctypes.c_float,
                                             ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_size_t,
                                             ctypes.POINTER(SmlaDims), vp]
    lib.sparse_mla_prefill_single_pass.restype = ctypes.c_int
    lib.sparse_mla_prefill_single_pass.argtypes = lib.sparse_mla_prefill_split.argtypes
    lib.sparse_mla_prefill_split_noalloc.restype = ctypes.c_int
    lib.sparse_mla_prefill_split_noalloc.argtypes = [vp, vp, vp, i32p, i32p, f32p, u32p, u32p, f32p,
                                                     ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.POINTER(SmlaDims), vp]
    lib.sparse_mla_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.sparse_mla_noalloc_scratch_bytes.argtypes = []
    lib.sparse_mla_split_workspace_bytes.restype = ctypes.c_size_t
    lib.sparse_mla_split_workspace_bytes.argtypes = [ctypes.POINTER(SmlaDims), ctypes.c_int32]
    lib.sparse_mla_auto_splits.restype = ctypes.c_int32
    lib.sparse_mla_auto_splits.argtypes = [ctypes.POINTER(SmlaDims), ctypes.c_int32]
    lib.sparse_mla_gather_debug.restype = ctypes.c_int
    lib.sparse_mla_gather_debug.argtypes = [vp, vp, i32p, i32p, u32p, u32p, ctypes.POINTER(SmlaDims), vp]
    ip = ctypes.POINTER(SmlaIndexDims)
    lib.sparse_mla_index_scores.restype = ctypes.c_int
    lib.sparse_mla_index_scores.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ip, vp]
    lib.sparse_mla_index_topk.restype = ctypes.c_int
    lib.sparse_mla_index_topk.argtypes = [vp, vp, vp, vp, vp, ip, vp]
    lib.mla_dense_prefill.restype = ctypes.c_int
    lib.mla_dense_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_int32,
                                      ctypes.POINTER(SmlaDenseDims), vp]
    lib.smla_status_string.restype = ctypes.c_char_p
    lib.smla_status_string.argtypes = [ctypes.c_int]
    lib.smla_version.restype = ctypes.c_int32
    lib.smla_version.argtypes = []
    if path is None:
        _lib = lib
    return lib


def _ptr(x: Optional[torch.Tensor]) -> Optional[int]:
    return None if x is None else x.data_ptr()


_INT32 = (torch.int32, torch.uint32) if hasattr(torch, "uint32") else (torch.int32,)


def _check(name: str, t: Optional[torch.Tensor], dtypes, shape, device, optional: bool = False) -> None:
    """Raise ValueError unless t is a contiguous tensor on `device` with one of
    `dtypes` and exactly `shape` (None entries match any size).  The library
    sizes every buffer from the dims it is given, so a tensor that is on the
    host, too small or of another element type would otherwise become an
    out-of-bounds device access instead of an error."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {tuple(dtypes)}")
    if len(shape) != t.dim() or any(w is not None and int(w) != int(n) for w, n in zip(shape, t.shape)):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_device(q: torch.Tensor, allow_cpu: bool):
    """The device every tensor of a call must share (a GPU unless the caller
    only validates arguments)."""
    if not isinstance(q, torch.Tensor):
        raise ValueError("expected a torch.Tensor")
    if q.device.type != "cuda" and not allow_cpu:
        raise ValueError(f"tensors must be on a GPU (got {q.device})")
    return q.device


def scale_columns(scale_block_size: int) -> int:
    """Columns of the scale table for a scale_block_size (0 when unit scale)."""
    sbs = int(scale_block_size)
    if sbs <= 0:
        return 0
    return 1 if sbs >= QK_DEPTH else (QK_DEPTH + sbs - 1) // sbs


def validate_prefill_args(q, kv_pages, page_table, cu_seqlens_q, indices, topk_lengths, scale_block_size=0,
                          scales=None, sink=None, out=None, allow_cpu=False):
    """Check every tensor sparse_mla_prefill passes to the C ABI (device,
    dtype, shape, contiguity); raises ValueError on the first mismatch."""
    dev = _check_device(q, allow_cpu)
    if q.dim() != 3:
        raise ValueError(f"q must be [T, H, {QK_DEPTH}]")
    T, H, _ = q.shape
    _check("q", q, (torch.bfloat16,), (None, None, QK_DEPTH), dev)
    if kv_pages is None or kv_pages.dim() != 3:
        raise ValueError(f"kv_pages must be [num_pages, page_size, {QK_DEPTH}]")
    _check("kv_pages", kv_pages, (torch.uint8, torch.float8_e4m3fn), (None, None, QK_DEPTH), dev)
    num_pages, P, _ = kv_pages.shape
    if page_table is None or page_table.dim() != 2:
        raise ValueError("page_table must be [B, max_pages]")
    _check("page_table", page_table, (torch.int32,), (None, None), dev)
    B = page_table.shape[0]
    _check("cu_seqlens_q", cu_seqlens_q, (torch.int32,), (B + 1,), dev)
    if indices is None or indices.dim() != 2:
        raise ValueError("indices must be [T, topk]")
    _check("indices", indices, _INT32, (T, None), dev)
    _check("topk_lengths", topk_lengths, _INT32, (T,), dev)
    ncols = scale_columns(scale_block_size)
    if int(scale_block_size) < 0:
        raise ValueError("scale_block_size must be >= 0")
    if ncols:  # unit scale (0): the library ignores scales
        _check("scales", scales, (torch.float32,), (num_pages * P, ncols), dev)
    _check("sink", sink, (torch.float32,), (H,), dev, optional=True)
    _check("out", out, (torch.bfloat16,), (T, H, V_DEPTH), dev, optional=True)


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def make_dims(q_or_T, H, topk, num_seqs, page_size, max_pages, num_pages) -> SmlaDims:
    d = SmlaDims()
    d.num_tokens = int(q_or_T)
    d.num_heads = int(H)
    d.qk_depth = QK_DEPTH
    d.v_depth = V_DEPTH
    d.topk = int(topk)
    d.num_seqs = int(num_seqs)
    d.page_size = int(page_size)
    d.max_pages_per_seq = int(max_pages)
    d.num_pages = int(num_pages)
    return d


def sparse_mla_prefill(q: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor,
                       cu_seqlens_q: torch.Tensor, indices: torch.Tensor, topk_lengths: torch.Tensor,
                       scale: float, scale_block_size: int = 0, scales: Optional[torch.Tensor] = None,
                       sink: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       stream=None, num_splits: int = 1,
                       workspace: Optional[torch.Tensor] = None, single_pass: bool = False) -> torch.Tensor:
    """Sparse MLA prefill attention through the C ABI.

    q bf16 [T, H, 576]; kv_pages uint8 (e4m3fn codes) [num_pages, P, 576];
    page_table int32 [B, max_pages]; cu_seqlens_q int32 [B + 1];
    indices int32/uint32 [T, K]; topk_lengths int32/uint32 [T];
    scales float32 [num_pages * P, ncols] or None; sink float32 [H] or None.
    num_splits: 1 calls sparse_mla_prefill; > 1 cuts each token's slots into
    that many runs (sparse_mla_prefill_split); 0 lets the library choose
    (sparse_mla_auto_splits).  workspace: a uint8 device tensor of at least
    split_workspace_bytes() bytes, allocated here when omitted.
    single_pass: call sparse_mla_prefill_single_pass instead (q and P as one
    FP8 operand each: faster, percent-level error; unit and per-row scales only).
    Returns out bf16 [T, H, 512] (written on `stream`).
    """
    validate_prefill_args(q, kv_pages, page_table, cu_seqlens_q, indices, topk_lengths, scale_block_size,
                          scales, sink, out)
    lib = load_library()
    T, H, D = q.shape
    num_pages, P, D2 = kv_pages.shape
    B, max_pages = page_table.shape
    K = indices.shape[1]
    if workspace is not None:
        _check("workspace", workspace, (torch.uint8,), (None,), q.device)
    if out is None:
        out = torch.empty((T, H, V_DEPTH), dtype=torch.bfloat16, device=q.device)
    dims = make_dims(T, H, K, B, P, max_pages, num_pages)
    if num_splits == 0:
        num_splits = int(lib.sparse_mla_auto_splits(ctypes.byref(dims), ctypes.c_int32(scale_block_size)))
    common = (_ptr(out), _ptr(q), _ptr(kv_pages), _ptr(page_table), _ptr(cu_seqlens_q), _ptr(scales),
              _ptr(indices), _ptr(topk_lengths), _ptr(sink), ctypes.c_float(scale),
              ctypes.c_int32(scale_block_size))
    if num_splits == 1 and not single_pass:
        st = lib.sparse_mla_prefill(*common, ctypes.byref(dims), _stream_handle(stream))
        what = "sparse_mla_prefill"
    else:
        need = int(lib.sparse_mla_split_workspace_bytes(ctypes.byref(dims), ctypes.c_int32(num_splits)))
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        fn = lib.sparse_mla_prefill_single_pass if single_pass else lib.sparse_mla_prefill_split
        wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        st = fn(*common, ctypes.c_int32(num_splits), _ptr(workspace), ctypes.c_size_t(wbytes),
                ctypes.byref(dims), _stream_handle(stream))
        what = "sparse_mla_prefill_single_pass" if single_pass else "sparse_mla_prefill_split"
    if st != SMLA_OK:
        raise SmlaError(st, what)
    return out


def sparse_mla_prefill_split_noalloc(q: torch.Tensor, kv_pages: torch.Tensor, page_table: torch.Tensor,
                                     cu_seqlens_q: torch.Tensor, indices: torch.Tensor, topk_lengths: torch.Tensor,
                                     scale: float, out: torch.Tensor, num_splits: int, scale_block_size: int = 0,
                                     scales: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None,
                                     stream=None) -> torch.Tensor:
    """sparse_mla_prefill_split without a workspace: the run partials go to the
    library's fixed per-GPU scratch array (noalloc_scratch_bytes() bytes).  The
    caller passes `out`; nothing is allocated here or in the library.  Calls
    that overlap on one GPU share the scratch array and race."""
    validate_prefill_args(q, kv_pages, page_table, cu_seqlens_q, indices, topk_lengths, scale_block_size,
                          scales, sink, out)
    if out is None:
        raise ValueError("out is required (this entry point allocates nothing)")
    lib = load_library()
    T, H, _ = q.shape
    num_pages, P, _ = kv_pages.shape
    B, max_pages = page_table.shape
    dims = make_dims(T, H, indices.shape[1], B, P, max_pages, num_pages)
    st = lib.sparse_mla_prefill_split_noalloc(_ptr(out), _ptr(q), _ptr(kv_pages), _ptr(page_table),
                                              _ptr(cu_seqlens_q), _ptr(scales), _ptr(indices), _ptr(topk_lengths),
                                              _ptr(sink), ctypes.c_float(scale), ctypes.c_int32(scale_block_size),
                                              ctypes.c_int32(num_splits), ctypes.byref(dims), _stream_handle(stream))
    if st != SMLA_OK:
        raise SmlaError(st, "sparse_mla_prefill_split_noalloc")
    return out


def noalloc_scratch_bytes() -> int:
    """Size of the fixed scratch array of sparse_mla_prefill_split_noalloc."""
    return int(load_library().sparse_mla_noalloc_scratch_bytes())


def split_workspace_bytes(T, H, topk, num_splits) -> int:
    """Workspace bytes of a split call with these sizes (0 when num_splits <= 1)."""
    dims = make_dims(T, H, topk, 1, 1, 1, 1)
    return int(load_library().sparse_mla_split_workspace_bytes(ctypes.byref(dims), ctypes.c_int32(num_splits)))


def auto_splits(T, H, topk, scale_block_size=0) -> int:
    """The library's run count for these sizes."""
    dims = make_dims(T, H, topk, 1, 1, 1, 1)
    return int(load_library().sparse_mla_auto_splits(ctypes.byref(dims), ctypes.c_int32(scale_block_size)))


def sparse_mla_gather_debug(kv_pages: torch.Tensor, page_table: torch.Tensor, cu_seqlens_q: torch.Tensor,
                            indices: torch.Tensor, topk_lengths: torch.Tensor, rows_out=None,
                            stream=None) -> torch.Tensor:
    """The gather stage alone: rows_out uint8 [T, K, 576] (zeros for slots not read)."""
    dev = _check_device(kv_pages, allow_cpu=False)
    _check("kv_pages", kv_pages, (torch.uint8, torch.float8_e4m3fn), (None, None, QK_DEPTH), dev)
    _check("page_table", page_table, (torch.int32,), (None, None), dev)
    _check("indices", indices, _INT32, (None, None), dev)
    T, K = indices.shape
    B = page_table.shape[0]
    _check("cu_seqlens_q", cu_seqlens_q, (torch.int32,), (B + 1,), dev)
    _check("topk_lengths", topk_lengths, _INT32, (T,), dev)
    _check("rows_out", rows_out, (torch.uint8,), (T, K, QK_DEPTH), dev, optional=True)
    lib = load_library()
    num_pages, P, _ = kv_pages.shape
    B, max_pages = page_table.shape
    if rows_out is None:
        rows_out = torch.empty((T, K, QK_DEPTH), dtype=torch.uint8, device=kv_pages.device)
    dims = make_dims(T, 0, K, B, P, max_pages, num_pages)
    st = lib.sparse_mla_gather_debug(_ptr(rows_out), _ptr(kv_pages), _ptr(page_table), _ptr(cu_seqlens_q),
                                     _ptr(indices), _ptr(topk_lengths), ctypes.byref(dims),
                                     _stream_handle(stream))
    if st != SMLA_OK:
        raise SmlaError(st, "sparse_mla_gather_debug")
    return rows_out


def make_index_dims(T, H, num_seqs, page_size, max_pages, num_pages, score_stride, topk) -> SmlaIndexDims:
    d = SmlaIndexDims()
    d.num_tokens = int(T)
    d.num_heads = int(H)
    d.depth = INDEX_DEPTH
    d.num_seqs = int(num_seqs)
    d.page_size = int(page_size)
    d.max_pages_per_seq = int(max_pages)
    d.num_pages = int(num_pages)
    d.score_stride = int(score_stride)
    d.topk = int(topk)
    return d


def validate_index_scores_args(q, q_scale, k_pages, k_scale, page_table, cu_seqlens_q, seq_lens_k, score_stride,
                               scores=None, allow_cpu=False):
    """Device, dtype, shape and contiguity of sparse_mla_index_scores'
    tensors; raises ValueError on the first mismatch."""
    dev = _check_device(q, allow_cpu)
    if q.dim() != 3:
        raise ValueError(f"q must be [T, H, {INDEX_DEPTH}]")
    T, H, _ = q.shape
    _check("q", q, (torch.uint8, torch.float8_e4m3fn), (None, None, INDEX_DEPTH), dev)
    _check("q_scale", q_scale, (torch.float32,), (T, H), dev)
    if k_pages is None or k_pages.dim() != 3:
        raise ValueError(f"k_pages must be [num_pages, page_size, {INDEX_DEPTH}]")
    _check("k_pages", k_pages, (torch.uint8, torch.float8_e4m3fn), (None, None, INDEX_DEPTH), dev)
    num_pages, P, _ = k_pages.shape
    _check("k_scale", k_scale, (torch.float32,), (num_pages * P,), dev)
    if page_table is None or page_table.dim() != 2:
        raise ValueError("page_table must be [B, max_pages]")
    _check("page_table", page_table, (torch.int32,), (None, None), dev)
    B = page_table.shape[0]
    _check("cu_seqlens_q", cu_seqlens_q, (torch.int32,), (B + 1,), dev)
    _check("seq_lens_k", seq_lens_k, (torch.int32,), (B,), dev)
    _check("scores", scores, (torch.float32,), (T, int(score_stride)), dev, optional=True)


def validate_index_topk_args(scores, cu_seqlens_q, seq_lens_k, topk, indices=None, topk_lengths=None,
                             allow_cpu=False):
    """The same for sparse_mla_index_topk."""
    dev = _check_device(scores, allow_cpu)
    if scores.dim() != 2:
        raise ValueError("scores must be [T, score_stride]")
    _check("scores", scores, (torch.float32,), (None, None), dev)
    T = scores.shape[0]
    if seq_lens_k is None or seq_lens_k.dim() != 1:
        raise ValueError("seq_lens_k must be [B]")
    _check("seq_lens_k", seq_lens_k, (torch.int32,), (None,), dev)
    _check("cu_seqlens_q", cu_seqlens_q, (torch.int32,), (seq_lens_k.shape[0] + 1,), dev)
    if int(topk) < 0:
        raise ValueError("topk must be >= 0")
    _check("indices", indices, _INT32, (T, max(int(topk), 1)), dev, optional=True)
    _check("topk_lengths", topk_lengths, _INT32, (T,), dev, optional=True)


def sparse_mla_index_scores(q: torch.Tensor, q_scale: torch.Tensor, k_pages: torch.Tensor,
                            k_scale: torch.Tensor, page_table: torch.Tensor, cu_seqlens_q: torch.Tensor,
                            seq_lens_k: torch.Tensor, score_stride: int, scores: Optional[torch.Tensor] = None,
                            topk: int = 0, stream=None) -> torch.Tensor:
    """Indexer score buffer through the C ABI.

    q uint8 (e4m3fn codes) [T, H, 128]; q_scale float32 [T, H];
    k_pages uint8 [num_pages, P, 128]; k_scale float32 [num_pages * P];
    page_table int32 [B, max_pages]; cu_seqlens_q int32 [B + 1]; seq_lens_k int32 [B].
    Returns scores float32 [T, score_stride] (-inf past each token's causal prefix).
    """
    validate_index_scores_args(q, q_scale, k_pages, k_scale, page_table, cu_seqlens_q, seq_lens_k, score_stride,
                               scores)
    lib = load_library()
    T, H, D = q.shape
    num_pages, P, _ = k_pages.shape
    B, max_pages = page_table.shape
    if scores is None:
        scores = torch.empty((T, score_stride), dtype=torch.float32, device=q.device)
    dims = make_index_dims(T, H, B, P, max_pages, num_pages, score_stride, topk)
    st = lib.sparse_mla_index_scores(_ptr(scores), _ptr(q), _ptr(q_scale), _ptr(k_pages), _ptr(k_scale),
                                     _ptr(page_table), _ptr(cu_seqlens_q), _ptr(seq_lens_k), ctypes.byref(dims),
                                     _stream_handle(stream))
    if st != SMLA_OK:
        raise SmlaError(st, "sparse_mla_index_scores")
    return scores


def sparse_mla_index_topk(scores: torch.Tensor, cu_seqlens_q: torch.Tensor, seq_lens_k: torch.Tensor, topk: int,
                          indices: Optional[torch.Tensor] = None, topk_lengths: Optional[torch.Tensor] = None,
                          stream=None):
    """Top-k of each score row through the C ABI.

    Returns (indices int32 [T, topk] holding uint32 patterns, ascending key
    order, 0xFFFFFFFF past the length; topk_lengths int32 [T]).
    """
    validate_index_topk_args(scores, cu_seqlens_q, seq_lens_k, topk, indices, topk_lengths)
    lib = load_library()
    T, stride = scores.shape
    B = seq_lens_k.shape[0]
    if indices is None:
        indices = torch.empty((T, max(topk, 1)), dtype=torch.int32, device=scores.device)
    if topk_lengths is None:
        topk_lengths = torch.empty((T,), dtype=torch.int32, device=scores.device)
    dims = make_index_dims(T, 32, B, 1, 1, 1, stride, topk)
    st = lib.sparse_mla_index_topk(_ptr(indices), _ptr(topk_lengths), _ptr(scores), _ptr(cu_seqlens_q),
                                   _ptr(seq_lens_k), ctypes.byref(dims), _stream_handle(stream))
    if st != SMLA_OK:
        raise SmlaError(st, "sparse_mla_index_topk")
    return indices[:, :topk], topk_lengths


def call_raw(**kwargs) -> int:
    """Call sparse_mla_prefill (with num_splits given, sparse_mla_prefill_split;
    with single_pass=True, sparse_mla_prefill_single_pass) with raw pointer / size arguments and return the status code (used to
    exercise the host-side argument checks)."""
    lib = load_library()
    dims = kwargs.pop("dims")
    args = [kwargs.get(k) for k in ("out", "q", "kv_pages", "page_table", "cu_seqlens_q", "scales",
                                    "indices", "topk_lengths", "sink")]
    args += [ctypes.c_float(kwargs.get("scale", 1.0)), ctypes.c_int32(kwargs.get("scale_block_size", 0))]
    dptr = ctypes.byref(dims) if dims is not None else None
    if kwargs.get("noalloc"):
        return lib.sparse_mla_prefill_split_noalloc(*args, ctypes.c_int32(kwargs.get("num_splits", 1)), dptr,
                                                    kwargs.get("stream"))
    if kwargs.get("single_pass"):
        return lib.sparse_mla_prefill_single_pass(*args, ctypes.c_int32(kwargs.get("num_splits", 1)),
                                                  kwargs.get("workspace"),
                                                  ctypes.c_size_t(kwargs.get("workspace_bytes", 0)), dptr,
                                                  kwargs.get("stream"))
    if "num_splits" in kwargs:
        return lib.sparse_mla_prefill_split(*args, ctypes.c_int32(kwargs["num_splits"]), kwargs.get("workspace"),
                                            ctypes.c_size_t(kwargs.get("workspace_bytes", 0)), dptr,
                                            kwargs.get("stream"))
    return lib.sparse_mla_prefill(*args, dptr, kwargs.get("stream"))


def version() -> int:
    return int(load_library().smla_version())


def status_string(code: int) -> str:
    return load_library().smla_status_string(code).decode()


def make_dense_dims(num_seqs, max_prompt_len, H, Hkv, page_size, max_pages, num_pages, causal=True,
                    nope_depth=128, rope_depth=64, v_depth=128) -> SmlaDenseDims:
    d = SmlaDenseDims()
    d.num_seqs = int(num_seqs)
    d.max_prompt_len = int(max_prompt_len)
    d.num_heads = int(H)
    d.num_kv_heads = int(Hkv)
    d.nope_depth = int(nope_depth)
    d.rope_depth = int(rope_depth)
    d.v_depth = int(v_depth)
    d.page_size = int(page_size)
    d.max_pages_per_seq = int(max_pages)
    d.num_pages = int(num_pages)
    d.causal = 1 if causal else 0
    return d


def validate_dense_args(q, k_nope, v, k_rope, k_rope_scales, page_table, valid_length, scale_block_size,
                        max_prompt_len, out=None, allow_cpu=False):
    """Device, dtype, shape and contiguity of mla_dense_prefill's tensors;
    raises ValueError on the first mismatch."""
    dev = _check_device(q, allow_cpu)
    if k_nope is None or k_nope.dim() != 4:
        raise ValueError("k_nope must be [num_pages, page_size, kv_heads, 128]")
    _check("k_nope", k_nope, (torch.bfloat16,), (None, None, None, None), dev)
    num_pages, P, Hkv, Dn = k_nope.shape
    if page_table is None or page_table.dim() != 2:
        raise ValueError("page_table must be [B, max_pages]")
    _check("page_table", page_table, (torch.int32,), (None, None), dev)
    B = page_table.shape[0]
    if q.dim() != 3:
        raise ValueError("q must be [B * S, H, nope + 64]")
    H = q.shape[1]
    _check("q", q, (torch.bfloat16,), (B * int(max_prompt_len), H, Dn + 64), dev)
    _check("v", v, (torch.bfloat16,), (num_pages, P, Hkv, None), dev)
    _check("k_rope", k_rope, (torch.uint8, torch.float8_e4m3fn), (num_pages, P, 64), dev)
    sbs = int(scale_block_size)
    if sbs < 0:
        raise ValueError("scale_block_size must be >= 0")
    ncols = 0 if sbs == 0 else (1 if sbs >= 64 else (64 + sbs - 1) // sbs)
    if ncols:  # unit scale (0): the library ignores k_rope_scales
        _check("k_rope_scales", k_rope_scales, (torch.float32,), (num_pages * P, ncols), dev)
    _check("valid_length", valid_length, _INT32, (B,), dev)
    _check("out", out, (torch.bfloat16,), (B * int(max_prompt_len), H, v.shape[3]), dev, optional=True)


def mla_dense_prefill(q: torch.Tensor, k_nope: torch.Tensor, v: torch.Tensor, k_rope: torch.Tensor,
                      k_rope_scales: Optional[torch.Tensor], page_table: torch.Tensor, valid_length: torch.Tensor,
                      scale: float, scale_block_size: int, max_prompt_len: int, causal: bool = True,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Dense MLA prefill with a block-scaled FP8 K_rope through the C ABI.

    q bf16 [B * S, H, 192]; k_nope, v bf16 [num_pages, P, Hkv, 128];
    k_rope uint8 (e4m3fn codes) [num_pages, P, 64]; k_rope_scales float32
    [num_pages * P, ncols] or None; page_table int32 [B, max_pages];
    valid_length int32 [B] (uint32 patterns).  Returns out bf16 [B * S, H, 128].
    """
    validate_dense_args(q, k_nope, v, k_rope, k_rope_scales, page_table, valid_length, scale_block_size,
                        max_prompt_len, out)
    lib = load_library()
    BS, H, DQ = q.shape
    num_pages, P, Hkv, Dn = k_nope.shape
    B, max_pages = page_table.shape
    if out is None:
        out = torch.empty((BS, H, v.shape[3]), dtype=torch.bfloat16, device=q.device)
    dims = make_dense_dims(B, max_prompt_len, H, Hkv, P, max_pages, num_pages, causal, Dn, 64, v.shape[3])
    st = lib.mla_dense_prefill(_ptr(out), _ptr(q), _ptr(k_nope), _ptr(v), _ptr(k_rope), _ptr(k_rope_scales),
                               _ptr(page_table), _ptr(valid_length), ctypes.c_float(scale),
                               int(scale_block_size), ctypes.byref(dims), _stream_handle(stream))
    if st != SMLA_OK:
        raise SmlaError(st, "mla_dense_prefill")
    return out
