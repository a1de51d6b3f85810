"""ctypes binding of libssa_peaks.so (include/ssa_peaks.h): measured machine
peaks, read beside the attention kernels' rates.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssa_peaks.so")
EXPORTS = ("ssa_peak_mfma", "ssa_peak_tile", "ssa_peak_read", "ssa_peak_copy", "ssa_peak_clock")
FLOP_PER_MFMA = 2 * 32 * 32 * 16     # v_mfma_f32_32x32x16_bf16
MFMA_PER_ITER = 16
MFMA_PER_TILE = 32                   # 16 score products + 16 P.V products
REALTIME_HZ = 100e6

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libssa_peaks.so not found at {path}; build it with "
                           "`python -m block_sparse_attention_kv_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz, i32, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_uint32
    lib.ssa_peak_mfma.argtypes = [i32, i32, vp, vp]
    lib.ssa_peak_tile.argtypes = [i32, i32, vp, vp]
    lib.ssa_peak_read.argtypes = [vp, sz, vp, i32, vp]
    lib.ssa_peak_copy.argtypes = [vp, vp, sz, i32, vp]
    lib.ssa_peak_clock.argtypes = [u32, vp, vp]
    for fn in EXPORTS:
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        raise RuntimeError(f"{fn} failed with status {status}")


def mfma(iters: int, n_blocks: int, out: torch.Tensor, stream=None):
    """Matrix-instruction loop; ``out`` is uint32-sized int32 [n_blocks * 16]."""
    assert out.is_cuda and out.dtype == torch.int32 and out.numel() >= 16 * n_blocks
    _check("ssa_peak_mfma", load_library().ssa_peak_mfma(iters, n_blocks, ctypes.c_void_p(out.data_ptr()),
                                                         _stream(stream)))


def tile(tiles: int, n_blocks: int, out: torch.Tensor, stream=None):
    """Compute-only attention-tile replica; ``out`` is uint32-sized int32 [n_blocks * 16]."""
    assert out.is_cuda and out.dtype == torch.int32 and out.numel() >= 16 * n_blocks
    _check("ssa_peak_tile", load_library().ssa_peak_tile(tiles, n_blocks, ctypes.c_void_p(out.data_ptr()),
                                                         _stream(stream)))


def read(src: torch.Tensor, out: torch.Tensor, n_blocks: int, stream=None):
    assert src.is_cuda and out.is_cuda and out.dtype == torch.int32 and out.numel() >= n_blocks
    nbytes = src.numel() * src.element_size()
    _check("ssa_peak_read", load_library().ssa_peak_read(ctypes.c_void_p(src.data_ptr()), nbytes,
                                                         ctypes.c_void_p(out.data_ptr()), n_blocks, _stream(stream)))


def copy(src: torch.Tensor, dst: torch.Tensor, n_blocks: int, stream=None):
    nbytes = src.numel() * src.element_size()
    assert src.is_cuda and dst.is_cuda and dst.numel() * dst.element_size() >= nbytes
    _check("ssa_peak_copy", load_library().ssa_peak_copy(ctypes.c_void_p(src.data_ptr()),
                                                         ctypes.c_void_p(dst.data_ptr()), nbytes, n_blocks,
                                                         _stream(stream)))


def clock(ticks: int, out: torch.Tensor, stream=None):
    """One wavefront records shader cycles over ``ticks`` real-time ticks; ``out`` int32 [2]."""
    assert out.is_cuda and out.dtype == torch.int32 and out.numel() >= 2
    _check("ssa_peak_clock", load_library().ssa_peak_clock(ticks, ctypes.c_void_p(out.data_ptr()),
                                                           _stream(stream)))
