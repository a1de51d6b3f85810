"""Thin Python binding of libssa (ctypes).  Argument marshalling only.

Every function takes device tensors, allocates its outputs with ``torch.empty``
on the same device, and calls the C-ABI entry point of the same name on the
current HIP stream.  All computation happens in the HIP kernels of libssa;
there is no CPU fallback: a missing library or a non-GPU tensor raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SSA_LIBRARY overrides the in-tree build (e.g. the host-ASan build of the same sources)
LIB_PATH = os.environ.get("SSA_LIBRARY") or os.path.join(_PKG, "libssa.so")

SSA_OK, SSA_ERR_INVALID_ARG, SSA_ERR_UNSUPPORTED, SSA_ERR_HIP, SSA_ERR_WORKSPACE = range(5)
SSA_OP_BLOCK_SCORES, SSA_OP_SELECT_TOPK, SSA_OP_SPARSE_FWD, SSA_OP_FULL_FWD, SSA_OP_SPARSE_BWD, SSA_OP_FULL_BWD = range(6)

EXPORTED_SYMBOLS = (
    "ssa_block_summaries", "ssa_block_scores", "ssa_select_topk", "ssa_block_sparse_attn_fwd",
    "ssa_full_attn_fwd_dropped_mass", "ssa_select_topk_shared", "ssa_block_sparse_attn_fwd_shared",
    "ssa_full_attn_fwd_dropped_mass_shared", "ssa_block_sparse_attn_fwd_early_stop", "ssa_block_sparse_attn_bwd",
    "ssa_block_sparse_attn_bwd_shared", "ssa_full_attn_bwd", "ssa_block_summaries_learned", "ssa_entmax_route",
    "ssa_block_sparse_attn_fwd_biased", "ssa_block_sparse_attn_fwd_noalloc", "ssa_decode_scores_select",
    "ssa_workspace_bytes",
    "ssa_status_string",
    "ssa_last_error", "ssa_version",
)


class Shape(ctypes.Structure):
    """Mirror of ``ssa_shape_t``."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("seq_q", ctypes.c_int32), ("seq_kv", ctypes.c_int32), ("q_offset", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
    ]

    def __repr__(self):
        return "Shape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class SSAError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


_lib_handle = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libssa.so (built in-tree).  Raises if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(path):
        raise RuntimeError(
            f"libssa.so not found at {path}; build it with "
            "`python -m block_sparse_attention_kv_amd.build` (there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    sp = ctypes.POINTER(Shape)
    lib.ssa_block_summaries.argtypes = [sp, vp, vp, vp]
    lib.ssa_block_scores.argtypes = [sp, vp, vp, vp, ctypes.c_int, vp, vp]
    lib.ssa_select_topk.argtypes = [sp, vp, vp, vp]
    lib.ssa_block_sparse_attn_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssa_full_attn_fwd_dropped_mass.argtypes = [sp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.ssa_select_topk_shared.argtypes = [sp, vp, vp, vp]
    lib.ssa_block_sparse_attn_fwd_shared.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssa_full_attn_fwd_dropped_mass_shared.argtypes = [sp, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.ssa_block_sparse_attn_fwd_early_stop.argtypes = [sp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp,
                                                         sz, vp]
    lib.ssa_block_sparse_attn_bwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssa_block_sparse_attn_bwd_shared.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssa_full_attn_bwd.argtypes = [sp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    f32 = ctypes.c_float
    lib.ssa_block_summaries_learned.argtypes = [sp, vp, vp, vp, vp]
    lib.ssa_entmax_route.argtypes = [sp, vp, f32, f32, f32, vp, vp, vp, vp]
    lib.ssa_block_sparse_attn_fwd_biased.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ssa_block_sparse_attn_fwd_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssa_decode_scores_select.argtypes = [sp, vp, vp, vp, vp, i32, vp]
    for fn in ("ssa_block_summaries", "ssa_block_scores", "ssa_select_topk",
               "ssa_block_sparse_attn_fwd", "ssa_full_attn_fwd_dropped_mass", "ssa_select_topk_shared",
               "ssa_block_sparse_attn_fwd_shared", "ssa_full_attn_fwd_dropped_mass_shared",
               "ssa_block_sparse_attn_fwd_early_stop", "ssa_block_sparse_attn_bwd",
               "ssa_block_sparse_attn_bwd_shared", "ssa_full_attn_bwd", "ssa_block_summaries_learned",
               "ssa_entmax_route", "ssa_block_sparse_attn_fwd_biased", "ssa_block_sparse_attn_fwd_noalloc",
               "ssa_decode_scores_select"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.ssa_workspace_bytes.argtypes = [sp, ctypes.c_int]
    lib.ssa_workspace_bytes.restype = ctypes.c_size_t
    lib.ssa_status_string.argtypes = [ctypes.c_int]
    lib.ssa_status_string.restype = ctypes.c_char_p
    lib.ssa_last_error.argtypes = []
    lib.ssa_last_error.restype = ctypes.c_char_p
    lib.ssa_version.argtypes = []
    lib.ssa_version.restype = ctypes.c_int32
    _lib_handle = lib
    return lib


def _check(fn: str, status: int):
    if status != SSA_OK:
        lib = load_library()
        raise SSAError(fn, status, lib.ssa_last_error().decode() or lib.ssa_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_gpu(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("libssa operates on GPU tensors only (no CPU fallback)")
        if t is not None and not t.is_contiguous():
            raise ValueError("libssa expects contiguous tensors")


BF16, F32, I32, U8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8


def _validate(fn: str, **spec):
    """Check every given tensor's dtype, exact shape and device against what the
    entry point reads or writes for this Shape (spec: name -> (tensor or None,
    dtype, shape or None for any)), then that they are contiguous GPU tensors.
    A mismatch raises ValueError before anything reaches the library."""
    dev = None
    for name, (t, dtype, shp) in spec.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{fn}: {name} must be a torch.Tensor")
        if t.dtype != dtype:
            raise ValueError(f"{fn}: {name} has dtype {t.dtype}, expected {dtype}")
        if shp is not None and tuple(t.shape) != tuple(int(x) for x in shp):
            raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shp)}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{fn}: {name} is on {t.device}, the other tensors on {dev}")
    _require_gpu(*(t for t, _, _ in spec.values()))


def _dims(shape: "Shape"):
    """(b, Hq, Hkv, seq_q, seq_kv, d, nqb, nkb, topk) of a Shape."""
    return (shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.seq_q, shape.seq_kv, shape.head_dim,
            n_blocks(shape.seq_q, shape.block), n_blocks(shape.seq_kv, shape.block), shape.topk)


def _full_rows(shape: "Shape", q_block_begin: int, q_block_count: Optional[int]):
    nqb = n_blocks(shape.seq_q, shape.block)
    if q_block_count is None:
        q_block_count = nqb - q_block_begin
    rows = max(0, min(shape.seq_q, (q_block_begin + q_block_count) * shape.block) - q_block_begin * shape.block)
    return q_block_count, rows


def make_shape(q: torch.Tensor, kv_heads: int, seq_kv: int, *, block: int = 64, topk: int = 16,
               scale: float = 0.0, causal: int = 1) -> Shape:
    """Shape for Q [b, Hq, seq_q, d] against a K/V of ``seq_kv`` rows; the query
    rows are the last ``seq_q`` positions (q_offset = seq_kv - seq_q)."""
    b, hq, seq_q, d = q.shape
    return Shape(batch=b, n_q_heads=hq, n_kv_heads=kv_heads, seq_q=seq_q, seq_kv=seq_kv,
                 q_offset=seq_kv - seq_q, head_dim=d, block=block, topk=topk, causal=causal,
                 scale=float(scale))


def n_blocks(n: int, block: int) -> int:
    return -(-n // block)


def ssa_workspace_bytes(shape: Shape, op: int) -> int:
    return int(load_library().ssa_workspace_bytes(ctypes.byref(shape), op))


def ssa_block_summaries(k: torch.Tensor, *, block: int = 64) -> torch.Tensor:
    """Key-block summaries fp32 [b, Hkv, nkb, d] of bf16 K [b, Hkv, seq_kv, d]."""
    _validate("ssa_block_summaries", k=(k, BF16, None))
    if k.dim() != 4:
        raise ValueError(f"ssa_block_summaries: k must be [b, Hkv, seq_kv, d], got shape {tuple(k.shape)}")
    b, hkv, n, d = k.shape
    shape = Shape(batch=b, n_q_heads=hkv, n_kv_heads=hkv, seq_q=n, seq_kv=n, q_offset=0,
                  head_dim=d, block=block, topk=1, causal=1, scale=0.0)
    ks = torch.empty((b, hkv, n_blocks(n, block), d), dtype=torch.float32, device=k.device)
    _check("ssa_block_summaries", load_library().ssa_block_summaries(
        ctypes.byref(shape), _ptr(k), _ptr(ks), _stream(k.device)))
    return ks


def ssa_block_summaries_learned(k: torch.Tensor, qbar: torch.Tensor, *, block: int = 64, scale: float = 0.0,
                                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Chunk summaries fp32 [b, Hkv, nkb, d] from a learned query qbar fp32
    [Hkv, d] (softmax-weighted key average per block; scale 0 = 1/sqrt(d))."""
    if k.dim() != 4:
        raise ValueError(f"ssa_block_summaries_learned: k must be [b, Hkv, seq_kv, d], got shape {tuple(k.shape)}")
    b, hkv, n, d = k.shape
    _validate("ssa_block_summaries_learned", k=(k, BF16, None), qbar=(qbar, F32, (hkv, d)),
              out=(out, F32, (b, hkv, n_blocks(n, block), d)))
    shape = Shape(batch=b, n_q_heads=hkv, n_kv_heads=hkv, seq_q=n, seq_kv=n, q_offset=0,
                  head_dim=d, block=block, topk=1, causal=1, scale=float(scale))
    if out is None:
        out = torch.empty((b, hkv, n_blocks(n, block), d), dtype=torch.float32, device=k.device)
    _check("ssa_block_summaries_learned", load_library().ssa_block_summaries_learned(
        ctypes.byref(shape), _ptr(k), _ptr(qbar), _ptr(out), _stream(k.device)))
    return out


def ssa_entmax_route(shape: Shape, scores: torch.Tensor, alpha: float, gamma: float, sigma: float,
                     idx=None, bias=None, weights=None, with_weights: bool = True):
    """(block_idx int32 [b, Hkv, nqb, topk], block_bias fp32 [b, Hkv, nqb, topk],
    weights fp32 [b, Hkv, nqb, nkb] or None): alpha-entmax routing averaged over
    each KV group."""
    b_, hq_, hkv_, _, _, _, nqb_, nkb_, k_ = _dims(shape)
    _validate("ssa_entmax_route", scores=(scores, F32, (b_, hq_, nqb_, nkb_)), idx=(idx, I32, (b_, hkv_, nqb_, k_)),
              bias=(bias, F32, (b_, hkv_, nqb_, k_)), weights=(weights, F32, (b_, hkv_, nqb_, nkb_)))
    b, hkv = shape.batch, shape.n_kv_heads
    nqb, nkb = n_blocks(shape.seq_q, shape.block), n_blocks(shape.seq_kv, shape.block)
    if idx is None:
        idx = torch.empty((b, hkv, nqb, shape.topk), dtype=torch.int32, device=scores.device)
    if bias is None:
        bias = torch.empty((b, hkv, nqb, shape.topk), dtype=torch.float32, device=scores.device)
    if weights is None and with_weights:
        weights = torch.empty((b, hkv, nqb, nkb), dtype=torch.float32, device=scores.device)
    _check("ssa_entmax_route", load_library().ssa_entmax_route(
        ctypes.byref(shape), _ptr(scores), float(alpha), float(gamma), float(sigma), _ptr(idx), _ptr(bias),
        _ptr(weights), _stream(scores.device)))
    return idx, bias, weights


def ssa_block_sparse_attn_fwd_biased(shape: Shape, q, k, v, block_idx, block_bias, out=None, lse=None,
                                     workspace: Optional[torch.Tensor] = None):
    """(out bf16 [b, Hq, seq_q, d], lse fp32 [b, Hq, seq_q]) of the block-sparse
    forward over group-shared lists with a per-block logit bias (decode uses a
    workspace, allocated here when not given)."""
    b_, hq_, hkv_, sq_, skv_, d_, nqb_, _, k_ = _dims(shape)
    _validate("ssa_block_sparse_attn_fwd_biased", q=(q, BF16, (b_, hq_, sq_, d_)), k=(k, BF16, (b_, hkv_, skv_, d_)),
              v=(v, BF16, (b_, hkv_, skv_, d_)), block_idx=(block_idx, I32, (b_, hkv_, nqb_, k_)),
              block_bias=(block_bias, F32, (b_, hkv_, nqb_, k_)), out=(out, BF16, (b_, hq_, sq_, d_)),
              lse=(lse, F32, (b_, hq_, sq_)), workspace=(workspace, U8, None))
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    need = ssa_workspace_bytes(shape, SSA_OP_SPARSE_FWD)
    if workspace is None and need > 0:
        workspace = torch.zeros((need,), dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("ssa_block_sparse_attn_fwd_biased", load_library().ssa_block_sparse_attn_fwd_biased(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(block_bias), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(q.device)))
    return out, lse


def ssa_block_scores(shape: Shape, q: torch.Tensor, k: Optional[torch.Tensor] = None,
                     k_summary: Optional[torch.Tensor] = None, *, summary_out: Optional[torch.Tensor] = None,
                     scores: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(scores [b, Hq, nqb, nkb] fp32, k_summary).  With ``k_summary`` given the
    cached summaries are used (K may be None); otherwise they are computed from K
    (into ``summary_out`` when given)."""
    b_, hq_, hkv_, sq_, skv_, d_, nqb_, nkb_, _ = _dims(shape)
    _validate("ssa_block_scores", q=(q, BF16, (b_, hq_, sq_, d_)), k=(k, BF16, (b_, hkv_, skv_, d_)),
              k_summary=(k_summary, F32, (b_, hkv_, nkb_, d_)), summary_out=(summary_out, F32, (b_, hkv_, nkb_, d_)),
              scores=(scores, F32, (b_, hq_, nqb_, nkb_)))
    if k is None and k_summary is None:
        raise ValueError("ssa_block_scores: give k or k_summary")
    summary_is_input = k_summary is not None
    if not summary_is_input:
        k_summary = summary_out if summary_out is not None else torch.empty(
            (shape.batch, shape.n_kv_heads, n_blocks(shape.seq_kv, shape.block), shape.head_dim),
            dtype=torch.float32, device=q.device)
    if scores is None:
        scores = torch.empty((shape.batch, shape.n_q_heads, n_blocks(shape.seq_q, shape.block),
                              n_blocks(shape.seq_kv, shape.block)), dtype=torch.float32, device=q.device)
    _check("ssa_block_scores", load_library().ssa_block_scores(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(k_summary), int(summary_is_input), _ptr(scores),
        _stream(q.device)))
    return scores, k_summary


def ssa_select_topk(shape: Shape, scores: torch.Tensor, idx: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Selected key blocks int32 [b, Hq, nqb, topk], ascending, -1 padded."""
    b_, hq_, _, _, _, _, nqb_, nkb_, k_ = _dims(shape)
    _validate("ssa_select_topk", scores=(scores, F32, (b_, hq_, nqb_, nkb_)), idx=(idx, I32, (b_, hq_, nqb_, k_)))
    if idx is None:
        idx = torch.empty((shape.batch, shape.n_q_heads, n_blocks(shape.seq_q, shape.block), shape.topk),
                          dtype=torch.int32, device=scores.device)
    _check("ssa_select_topk", load_library().ssa_select_topk(
        ctypes.byref(shape), _ptr(scores), _ptr(idx), _stream(scores.device)))
    return idx


def ssa_select_topk_shared(shape: Shape, scores: torch.Tensor, idx: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Group-shared selection int32 [b, Hkv, nqb, topk] from the mean of each
    KV group's per-head scores."""
    b_, hq_, hkv_, _, _, _, nqb_, nkb_, k_ = _dims(shape)
    _validate("ssa_select_topk_shared", scores=(scores, F32, (b_, hq_, nqb_, nkb_)),
              idx=(idx, I32, (b_, hkv_, nqb_, k_)))
    if idx is None:
        idx = torch.empty((shape.batch, shape.n_kv_heads, n_blocks(shape.seq_q, shape.block), shape.topk),
                          dtype=torch.int32, device=scores.device)
    _check("ssa_select_topk_shared", load_library().ssa_select_topk_shared(
        ctypes.byref(shape), _ptr(scores), _ptr(idx), _stream(scores.device)))
    return idx


def ssa_decode_scores_select(shape: Shape, q, k_summary, scores: Optional[torch.Tensor] = None,
                             idx: Optional[torch.Tensor] = None, shared: bool = False, with_scores: bool = True):
    """Decode scores and top-k selection in one launch: (scores fp32 [b, Hq, 1, nkb]
    or None, idx int32 [b, Hq or Hkv, 1, topk]).  ``with_scores=False`` skips
    writing the scores."""
    b_, hq_, hkv_, sq_, _, d_, nqb_, nkb_, k_ = _dims(shape)
    _validate("ssa_decode_scores_select", q=(q, BF16, (b_, hq_, sq_, d_)), k_summary=(k_summary, F32, (b_, hkv_, nkb_, d_)),
              scores=(scores, F32, (b_, hq_, nqb_, nkb_)), idx=(idx, I32, (b_, hkv_ if shared else hq_, nqb_, k_)))
    if scores is None and with_scores:
        scores = torch.empty((b_, hq_, nqb_, nkb_), dtype=torch.float32, device=q.device)
    if idx is None:
        idx = torch.empty((b_, hkv_ if shared else hq_, nqb_, k_), dtype=torch.int32, device=q.device)
    _check("ssa_decode_scores_select", load_library().ssa_decode_scores_select(
        ctypes.byref(shape), _ptr(q), _ptr(k_summary), _ptr(scores), _ptr(idx), 1 if shared else 0,
        _stream(q.device)))
    return scores, idx


def ssa_block_sparse_attn_fwd(shape: Shape, q, k, v, block_idx, workspace: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                              shared: bool = False):
    """(out bf16 [b, Hq, seq_q, d], lse fp32 [b, Hq, seq_q]).  ``shared``: block_idx
    is a group-shared selection [b, Hkv, nqb, topk] (ssa_block_sparse_attn_fwd_shared).  ``workspace``
    (zero-filled before first use; every call leaves its work queue zero) is
    allocated when not given."""
    b_, hq_, hkv_, sq_, skv_, d_, nqb_, _, k_ = _dims(shape)
    _validate("ssa_block_sparse_attn_fwd", q=(q, BF16, (b_, hq_, sq_, d_)), k=(k, BF16, (b_, hkv_, skv_, d_)),
              v=(v, BF16, (b_, hkv_, skv_, d_)), block_idx=(block_idx, I32, (b_, hkv_ if shared else hq_, nqb_, k_)),
              workspace=(workspace, U8, None), out=(out, BF16, (b_, hq_, sq_, d_)), lse=(lse, F32, (b_, hq_, sq_)))
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    need = ssa_workspace_bytes(shape, SSA_OP_SPARSE_FWD)
    if workspace is None and need > 0:
        workspace = torch.zeros((need,), dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    name = "ssa_block_sparse_attn_fwd_shared" if shared else "ssa_block_sparse_attn_fwd"
    _check(name, getattr(load_library(), name)(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(q.device)))
    return out, lse


def ssa_block_sparse_attn_fwd_noalloc(shape: Shape, q, k, v, block_idx, out: torch.Tensor, lse: torch.Tensor):
    """ssa_block_sparse_attn_fwd with the library's static scratch array as
    workspace: the caller passes the outputs and nothing is allocated."""
    if out is None or lse is None:
        raise ValueError("ssa_block_sparse_attn_fwd_noalloc: out and lse are required")
    b_, hq_, hkv_, sq_, skv_, d_, nqb_, _, k_ = _dims(shape)
    _validate("ssa_block_sparse_attn_fwd_noalloc", q=(q, BF16, (b_, hq_, sq_, d_)),
              k=(k, BF16, (b_, hkv_, skv_, d_)), v=(v, BF16, (b_, hkv_, skv_, d_)),
              block_idx=(block_idx, I32, (b_, hq_, nqb_, k_)), out=(out, BF16, (b_, hq_, sq_, d_)),
              lse=(lse, F32, (b_, hq_, sq_)))
    _check("ssa_block_sparse_attn_fwd_noalloc", load_library().ssa_block_sparse_attn_fwd_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(out), _ptr(lse), _stream(q.device)))
    return out, lse


def ssa_full_attn_fwd_dropped_mass(shape: Shape, q, k, v, block_idx, q_block_begin: int = 0,
                                   q_block_count: Optional[int] = None, out=None, lse=None, dropped=None,
                                   shared: bool = False, workspace: Optional[torch.Tensor] = None):
    """(out_full bf16, lse_full fp32, dropped_mass fp32) over query blocks
    [q_block_begin, q_block_begin + q_block_count).  ``shared``: block_idx is a
    group-shared selection (ssa_full_attn_fwd_dropped_mass_shared).  ``workspace``
    (zero-filled before first use; every call leaves it zero) holds the work
    queue; one is allocated when not given."""
    q_block_count, rows = _full_rows(shape, q_block_begin, q_block_count)
    b_, hq_, hkv_, sq_, skv_, d_, nqb_, _, k_ = _dims(shape)
    _validate("ssa_full_attn_fwd_dropped_mass", q=(q, BF16, (b_, hq_, sq_, d_)), k=(k, BF16, (b_, hkv_, skv_, d_)),
              v=(v, BF16, (b_, hkv_, skv_, d_)), block_idx=(block_idx, I32, (b_, hkv_ if shared else hq_, nqb_, k_)),
              out=(out, BF16, (b_, hq_, rows, d_)), lse=(lse, F32, (b_, hq_, rows)),
              dropped=(dropped, F32, (b_, hq_, rows)), workspace=(workspace, U8, None))
    b, hq, d = shape.batch, shape.n_q_heads, shape.head_dim
    if out is None:
        out = torch.empty((b, hq, rows, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((b, hq, rows), dtype=torch.float32, device=q.device)
    if dropped is None:
        dropped = torch.empty((b, hq, rows), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.zeros((max(1, ssa_workspace_bytes(shape, SSA_OP_FULL_FWD)),), dtype=torch.uint8,
                                device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    name = "ssa_full_attn_fwd_dropped_mass_shared" if shared else "ssa_full_attn_fwd_dropped_mass"
    _check(name, getattr(load_library(), name)(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), int(q_block_begin),
        int(q_block_count), _ptr(out), _ptr(lse), _ptr(dropped), _ptr(workspace), ws_bytes, _stream(q.device)))
    return out, lse, dropped


def ssa_block_sparse_attn_fwd_early_stop(shape: Shape, q, k, v, scores, block_idx, tau: float, out=None, lse=None,
                                         blocks_used=None):
    """(out bf16 [b, Hq, seq_q, d], lse fp32 [b, Hq, seq_q], blocks_used int32 [b, Hq, nqb])."""
    b_, hq_, hkv_, sq_, skv_, d_, nqb_, nkb_, k_ = _dims(shape)
    _validate("ssa_block_sparse_attn_fwd_early_stop", q=(q, BF16, (b_, hq_, sq_, d_)),
              k=(k, BF16, (b_, hkv_, skv_, d_)), v=(v, BF16, (b_, hkv_, skv_, d_)),
              scores=(scores, F32, (b_, hq_, nqb_, nkb_)), block_idx=(block_idx, I32, (b_, hq_, nqb_, k_)),
              out=(out, BF16, (b_, hq_, sq_, d_)), lse=(lse, F32, (b_, hq_, sq_)),
              blocks_used=(blocks_used, I32, (b_, hq_, nqb_)))
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if blocks_used is None:
        blocks_used = torch.empty((shape.batch, shape.n_q_heads, n_blocks(shape.seq_q, shape.block)),
                                  dtype=torch.int32, device=q.device)
    _check("ssa_block_sparse_attn_fwd_early_stop", load_library().ssa_block_sparse_attn_fwd_early_stop(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(scores), _ptr(block_idx), float(tau), _ptr(out),
        _ptr(lse), _ptr(blocks_used), None, 0, _stream(q.device)))
    return out, lse, blocks_used


def _bwd_outputs(shape: Shape, q, rows: int, dq, dk, dv, workspace, op: int):
    b, hq, hkv, d = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    if dq is None:
        dq = torch.empty((b, hq, rows, d), dtype=torch.bfloat16, device=q.device)
    if dk is None:
        dk = torch.empty((b, hkv, shape.seq_kv, d), dtype=torch.bfloat16, device=q.device)
    if dv is None:
        dv = torch.empty((b, hkv, shape.seq_kv, d), dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        workspace = torch.empty((max(1, ssa_workspace_bytes(shape, op)),), dtype=torch.uint8, device=q.device)
    return dq, dk, dv, workspace, workspace.numel() * workspace.element_size()


def ssa_block_sparse_attn_bwd(shape: Shape, q, k, v, block_idx, out, lse, dout, dq=None, dk=None, dv=None,
                              workspace: Optional[torch.Tensor] = None, shared: bool = False):
    """(dq bf16 [b, Hq, seq_q, d], dk, dv bf16 [b, Hkv, seq_kv, d]): gradients of
    sum(dout * out) for the block-sparse forward that produced out and lse.
    ``shared``: block_idx is a group-shared selection (ssa_block_sparse_attn_bwd_shared)."""
    b_, hq_, hkv_, sq_, skv_, d_, nqb_, _, k_ = _dims(shape)
    _validate("ssa_block_sparse_attn_bwd", q=(q, BF16, (b_, hq_, sq_, d_)), k=(k, BF16, (b_, hkv_, skv_, d_)),
              v=(v, BF16, (b_, hkv_, skv_, d_)), block_idx=(block_idx, I32, (b_, hkv_ if shared else hq_, nqb_, k_)),
              out=(out, BF16, (b_, hq_, sq_, d_)), lse=(lse, F32, (b_, hq_, sq_)), dout=(dout, BF16, (b_, hq_, sq_, d_)),
              dq=(dq, BF16, (b_, hq_, sq_, d_)), dk=(dk, BF16, (b_, hkv_, skv_, d_)), dv=(dv, BF16, (b_, hkv_, skv_, d_)),
              workspace=(workspace, U8, None))
    dq, dk, dv, workspace, ws_bytes = _bwd_outputs(shape, q, shape.seq_q, dq, dk, dv, workspace, SSA_OP_SPARSE_BWD)
    name = "ssa_block_sparse_attn_bwd_shared" if shared else "ssa_block_sparse_attn_bwd"
    _check(name, getattr(load_library(), name)(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(out), _ptr(lse), _ptr(dout),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, _stream(q.device)))
    return dq, dk, dv


def ssa_full_attn_bwd(shape: Shape, q, k, v, out_full, lse_full, dout_full, q_block_begin: int = 0,
                      q_block_count: Optional[int] = None, dq=None, dk=None, dv=None,
                      workspace: Optional[torch.Tensor] = None):
    """(dq bf16 [b, Hq, rows, d], dk, dv bf16 [b, Hkv, seq_kv, d]): gradients of
    sum(dout_full * out_full) for the full causal forward over query blocks
    [q_block_begin, q_block_begin + q_block_count)."""
    q_block_count, rows = _full_rows(shape, q_block_begin, q_block_count)
    b_, hq_, hkv_, sq_, skv_, d_, _, _, _ = _dims(shape)
    _validate("ssa_full_attn_bwd", q=(q, BF16, (b_, hq_, sq_, d_)), k=(k, BF16, (b_, hkv_, skv_, d_)),
              v=(v, BF16, (b_, hkv_, skv_, d_)), out_full=(out_full, BF16, (b_, hq_, rows, d_)),
              lse_full=(lse_full, F32, (b_, hq_, rows)), dout_full=(dout_full, BF16, (b_, hq_, rows, d_)),
              dq=(dq, BF16, (b_, hq_, rows, d_)), dk=(dk, BF16, (b_, hkv_, skv_, d_)),
              dv=(dv, BF16, (b_, hkv_, skv_, d_)), workspace=(workspace, U8, None))
    dq, dk, dv, workspace, ws_bytes = _bwd_outputs(shape, q, rows, dq, dk, dv, workspace, SSA_OP_FULL_BWD)
    _check("ssa_full_attn_bwd", load_library().ssa_full_attn_bwd(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), int(q_block_begin), int(q_block_count), _ptr(out_full),
        _ptr(lse_full), _ptr(dout_full), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
        _stream(q.device)))
    return dq, dk, dv


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
