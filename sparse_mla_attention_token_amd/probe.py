"""ctypes binding of the measurement probes (include/smla_probe.h,
libsmla_probe.so): the measured matrix-core peak of the MFMA shapes the
attention uses, and the rate of its row gather.  Argument marshalling only."""

from __future__ import annotations

import ctypes
import os
from pathlib import Path
from typing import Optional

import torch

_PKG = Path(__file__).resolve().parent
PROBE_LIB_PATH = Path(os.environ.get("SMLA_PROBE_LIB", _PKG / "libsmla_probe.so"))

PROBE_SYMBOLS = ("smla_probe_mfma", "smla_probe_mfma_flop", "smla_probe_gather", "smla_probe_coexec")
MFMA_KINDS = {"fp8": 0, "fp16": 1, "bf16": 2, "fp16_16x16": 3, "bf16_16x16": 4}

_lib = None


def load_probe_library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not PROBE_LIB_PATH.exists():
        raise ImportError(f"{PROBE_LIB_PATH} not found: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(str(PROBE_LIB_PATH))
    vp = ctypes.c_void_p
    lib.smla_probe_mfma.restype = ctypes.c_int
    lib.smla_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, vp, vp]
    lib.smla_probe_mfma_flop.restype = ctypes.c_int64
    lib.smla_probe_mfma_flop.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int]
    lib.smla_probe_gather.restype = ctypes.c_int
    lib.smla_probe_gather.argtypes = [vp, ctypes.c_uint64, vp, ctypes.c_int, ctypes.c_int, vp, vp]
    lib.smla_probe_coexec.restype = ctypes.c_int
    lib.smla_probe_coexec.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int, vp, vp, vp]
    _lib = lib
    return lib


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def mfma(kind: str, iters: int, blocks: int, out: torch.Tensor, stream=None) -> int:
    """Launch the back-to-back MFMA loop; returns the FLOP it performs."""
    lib = load_probe_library()
    k = MFMA_KINDS[kind]
    if out.dtype != torch.float32 or out.numel() < 4 * blocks or out.device.type != "cuda":
        raise ValueError("out must be a float32 GPU tensor of at least 4 * blocks elements")
    st = lib.smla_probe_mfma(k, int(iters), int(blocks), out.data_ptr(), _stream(stream))
    if st != 0:
        raise RuntimeError(f"smla_probe_mfma failed ({st})")
    return int(lib.smla_probe_mfma_flop(k, int(iters), int(blocks)))


def gather(pool: torch.Tensor, rows: torch.Tensor, tiles_per_block: int, blocks: int,
           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Launch the row-gather probe: rows uint32/int32 [blocks * tiles_per_block * 64]
    ids of 576-byte rows of pool (uint8, 16-byte aligned)."""
    lib = load_probe_library()
    if rows.numel() < blocks * tiles_per_block * 64 or rows.dtype not in (torch.int32, torch.uint32):
        raise ValueError("rows must hold blocks * tiles_per_block * 64 uint32 row ids")
    if pool.device != rows.device or pool.device.type != "cuda" or not pool.is_contiguous():
        raise ValueError("pool and rows must be contiguous GPU tensors on one device")
    if out is None:
        out = torch.empty(blocks, dtype=torch.int32, device=pool.device)
    st = lib.smla_probe_gather(pool.data_ptr(), pool.numel() * pool.element_size(), rows.data_ptr(),
                               int(tiles_per_block), int(blocks), out.data_ptr(), _stream(stream))
    if st != 0:
        raise RuntimeError(f"smla_probe_gather failed ({st})")
    return out


def coexec(mode: int, valu: int, iters: int, blocks: int, cycles: torch.Tensor, out: torch.Tensor,
           stream=None) -> None:
    """Launch the issue-behaviour probe (modes and counts as in smla_probe.h)."""
    lib = load_probe_library()
    if cycles.dtype != torch.int64 or cycles.numel() < 8 * blocks or cycles.device.type != "cuda":
        raise ValueError("cycles must be an int64 GPU tensor of at least 8 * blocks elements")
    if out.dtype != torch.float32 or out.numel() < 8 * blocks or out.device.type != "cuda":
        raise ValueError("out must be a float32 GPU tensor of at least 8 * blocks elements")
    st = lib.smla_probe_coexec(int(mode), int(valu), int(iters), int(blocks), cycles.data_ptr(), out.data_ptr(),
                               _stream(stream))
    if st != 0:
        raise RuntimeError(f"smla_probe_coexec failed ({st})")
