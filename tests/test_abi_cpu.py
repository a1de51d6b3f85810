"""CPU-side checks of the C-ABI library: it loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU runtime."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from block_sparse_attention_kv_amd import ssa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssa.h")
PEAKS_HEADER = os.path.join(ROOT, "include", "ssa_peaks.h")

FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10002)


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssa.LIB_PATH):
        from block_sparse_attention_kv_amd import build
        build.build()
    return ssa.load_library()


def good_shape(**kw):
    s = dict(batch=1, n_q_heads=4, n_kv_heads=2, seq_q=256, seq_kv=256, q_offset=0, head_dim=64,
             block=64, topk=2, causal=1, scale=0.0)
    s.update(kw)
    return ssa.Shape(**s)


def test_every_declared_symbol_is_exported(lib):
    declared = header_functions()
    assert set(declared) == set(ssa.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_peaks_library_exports_its_header():
    from block_sparse_attention_kv_amd import peaks
    if not os.path.exists(peaks.LIB_PATH):
        from block_sparse_attention_kv_amd import build
        build.build()
    plib = peaks.load_library()
    declared = header_functions(PEAKS_HEADER)
    assert set(declared) == set(peaks.EXPORTS)
    for name in declared:
        assert hasattr(plib, name), name
    # argument checks return before any launch
    assert plib.ssa_peak_mfma(0, 1, FAKE, None) == 1
    assert plib.ssa_peak_tile(0, 1, FAKE, None) == 1
    assert plib.ssa_peak_tile(1, 0, FAKE, None) == 1
    assert plib.ssa_peak_read(FAKE, 24, FAKE, 1, None) == 1
    assert plib.ssa_peak_copy(FAKE, MISALIGNED, 32, 1, None) == 1
    assert plib.ssa_peak_clock(0, FAKE, None) == 1


def test_version_and_status_strings(lib):
    assert lib.ssa_version() >= 10000
    for st in range(5):
        assert lib.ssa_status_string(st)
    assert lib.ssa_status_string(99) == b"unknown status"


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=3, n_kv_heads=2), ssa.SSA_ERR_INVALID_ARG),
    (dict(n_kv_heads=0), ssa.SSA_ERR_INVALID_ARG),
    (dict(seq_kv=255), ssa.SSA_ERR_INVALID_ARG),                     # seq_kv != q_offset + seq_q
    (dict(seq_q=100, seq_kv=132, q_offset=32), ssa.SSA_ERR_INVALID_ARG),  # chunk not block aligned
    (dict(topk=0), ssa.SSA_ERR_INVALID_ARG),
    (dict(batch=-1), ssa.SSA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), ssa.SSA_ERR_INVALID_ARG),
    (dict(head_dim=128), ssa.SSA_ERR_UNSUPPORTED),
    (dict(block=32), ssa.SSA_ERR_UNSUPPORTED),
    (dict(causal=0), ssa.SSA_ERR_UNSUPPORTED),
    (dict(topk=257), ssa.SSA_ERR_UNSUPPORTED),
    (dict(scale=-0.125), ssa.SSA_ERR_UNSUPPORTED),
])
def test_shape_validation(lib, kw, status):
    sh = good_shape(**kw)
    p = ctypes.byref(sh)
    assert lib.ssa_block_scores(p, FAKE, FAKE, FAKE, 0, FAKE, None) == status
    assert lib.ssa_select_topk(p, FAKE, FAKE, None) == status
    assert lib.ssa_block_sparse_attn_fwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == status
    assert lib.ssa_full_attn_fwd_dropped_mass(p, FAKE, FAKE, FAKE, FAKE, 0, 1, FAKE, FAKE, FAKE, None, 0,
                                              None) == status
    assert lib.ssa_select_topk_shared(p, FAKE, FAKE, None) == status
    assert lib.ssa_block_sparse_attn_fwd_shared(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == status
    assert lib.ssa_full_attn_fwd_dropped_mass_shared(p, FAKE, FAKE, FAKE, FAKE, 0, 1, FAKE, FAKE, FAKE, None, 0,
                                                     None) == status
    assert lib.ssa_block_sparse_attn_fwd_early_stop(p, FAKE, FAKE, FAKE, FAKE, FAKE, 0.01, FAKE, FAKE, FAKE, None,
                                                    0, None) == status
    assert lib.ssa_block_summaries_learned(p, FAKE, FAKE, FAKE, None) == status
    assert lib.ssa_entmax_route(p, FAKE, ctypes.c_float(1.5), ctypes.c_float(1.0), ctypes.c_float(1.0), FAKE, FAKE,
                                None, None) == status
    assert lib.ssa_block_sparse_attn_fwd_biased(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == status
    for fn in (lib.ssa_block_sparse_attn_bwd, lib.ssa_block_sparse_attn_bwd_shared):
        assert fn(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == status
    assert lib.ssa_full_attn_bwd(p, FAKE, FAKE, FAKE, 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                 None) == status
    assert lib.ssa_last_error()


def test_pointer_validation(lib):
    sh = good_shape()
    p = ctypes.byref(sh)
    assert lib.ssa_block_sparse_attn_fwd(p, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == ssa.SSA_ERR_INVALID_ARG
    assert b"q is NULL" in lib.ssa_last_error()
    assert lib.ssa_block_sparse_attn_fwd(p, MISALIGNED, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == ssa.SSA_ERR_INVALID_ARG
    assert b"aligned" in lib.ssa_last_error()
    assert lib.ssa_block_scores(p, FAKE, None, FAKE, 0, FAKE, None) == ssa.SSA_ERR_INVALID_ARG
    assert lib.ssa_select_topk(p, FAKE, None, None) == ssa.SSA_ERR_INVALID_ARG
    assert lib.ssa_select_topk_shared(p, None, FAKE, None) == ssa.SSA_ERR_INVALID_ARG
    assert lib.ssa_block_sparse_attn_fwd_shared(p, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 0,
                                                None) == ssa.SSA_ERR_INVALID_ARG
    assert b"block_idx is NULL" in lib.ssa_last_error()
    assert lib.ssa_block_summaries(None, FAKE, FAKE, None) == ssa.SSA_ERR_INVALID_ARG
    # query-block range outside the problem
    assert lib.ssa_full_attn_fwd_dropped_mass(p, FAKE, FAKE, FAKE, FAKE, 3, 2, FAKE, FAKE, FAKE, None, 0,
                                              None) == ssa.SSA_ERR_INVALID_ARG


def test_early_stop_threshold_validation(lib):
    p = ctypes.byref(good_shape())
    for tau in (-0.5, float("nan")):
        assert lib.ssa_block_sparse_attn_fwd_early_stop(p, FAKE, FAKE, FAKE, FAKE, FAKE, tau, FAKE, FAKE, FAKE, None,
                                                        0, None) == ssa.SSA_ERR_INVALID_ARG
        assert b"tau" in lib.ssa_last_error()
    assert lib.ssa_block_sparse_attn_fwd_early_stop(p, FAKE, FAKE, FAKE, None, FAKE, 0.1, FAKE, FAKE, FAKE, None,
                                                    0, None) == ssa.SSA_ERR_INVALID_ARG
    assert b"scores is NULL" in lib.ssa_last_error()


def test_noalloc_validation(lib):
    """The allocation-free forward validates like the workspace entry point and
    refuses a decode whose partials exceed its static array, all before any
    HIP call."""
    assert lib.ssa_block_sparse_attn_fwd_noalloc(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                 None) == ssa.SSA_ERR_INVALID_ARG
    p = ctypes.byref(good_shape())
    assert lib.ssa_block_sparse_attn_fwd_noalloc(p, FAKE, FAKE, MISALIGNED, FAKE, FAKE, FAKE,
                                                 None) == ssa.SSA_ERR_INVALID_ARG
    # 1024 sequences x 32 heads x 1 slice x 264 B = 8.65 MB > 8 MiB
    big = good_shape(batch=1024, n_q_heads=32, n_kv_heads=2, seq_q=1, seq_kv=128, q_offset=127, topk=2)
    assert lib.ssa_block_sparse_attn_fwd_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                 None) == ssa.SSA_ERR_WORKSPACE
    assert b"scratch" in lib.ssa_last_error()


def test_decode_scores_select_validation(lib):
    """The fused decode scoring + selection is decode only and refuses groups
    whose scores do not fit one workgroup, before any HIP call."""
    pre = good_shape()   # seq_q 256
    assert lib.ssa_decode_scores_select(ctypes.byref(pre), FAKE, FAKE, None, FAKE, 0, None) == ssa.SSA_ERR_INVALID_ARG
    big = good_shape(n_q_heads=64, n_kv_heads=1, seq_q=1, seq_kv=4096, q_offset=4095, topk=4)
    assert lib.ssa_decode_scores_select(ctypes.byref(big), FAKE, FAKE, None, FAKE, 0, None) == ssa.SSA_ERR_UNSUPPORTED
    long_ = good_shape(n_q_heads=32, n_kv_heads=2, seq_q=1, seq_kv=64 * 1024, q_offset=64 * 1024 - 1, topk=4)
    assert lib.ssa_decode_scores_select(ctypes.byref(long_), FAKE, FAKE, None, FAKE, 1, None) == ssa.SSA_ERR_UNSUPPORTED
    ok = good_shape(n_q_heads=32, n_kv_heads=2, seq_q=1, seq_kv=4096, q_offset=4095, topk=4)
    assert lib.ssa_decode_scores_select(ctypes.byref(ok), FAKE, FAKE, None, None, 0, None) == ssa.SSA_ERR_INVALID_ARG
    assert b"block_idx is NULL" in lib.ssa_last_error()


def test_decode_workspace(lib):
    sh = good_shape(batch=64, n_q_heads=32, n_kv_heads=2, seq_q=1, seq_kv=32768, q_offset=32767, topk=17)
    need = lib.ssa_workspace_bytes(ctypes.byref(sh), ssa.SSA_OP_SPARSE_FWD)
    assert need == 64 * 32 * 8 * 66 * 4        # 8 slices per KV group, (max, sum, o[64]) per head each
    # prefill: the optional work queue of the persistent launches (8 counters, one 128-byte line each)
    assert lib.ssa_workspace_bytes(ctypes.byref(sh), ssa.SSA_OP_FULL_FWD) == 1024
    assert lib.ssa_workspace_bytes(ctypes.byref(good_shape()), ssa.SSA_OP_SPARSE_FWD) == 1024
    assert lib.ssa_workspace_bytes(ctypes.byref(good_shape(head_dim=8)), ssa.SSA_OP_SPARSE_FWD) == 2**64 - 1
    # too small a workspace is refused before launch
    assert lib.ssa_block_sparse_attn_fwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 4,
                                         None) == ssa.SSA_ERR_WORKSPACE
    # decode lists beyond 2048 (heads per KV head x topk) are not implemented
    wide = good_shape(batch=1, n_q_heads=32, n_kv_heads=2, seq_q=1, seq_kv=64 * 300, q_offset=64 * 300 - 1, topk=200)
    assert lib.ssa_block_sparse_attn_fwd(ctypes.byref(wide), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                         None) == ssa.SSA_ERR_UNSUPPORTED
    # decode groups beyond 32 query heads per KV head are not implemented
    big = good_shape(batch=1, n_q_heads=64, n_kv_heads=1, seq_q=1, seq_kv=100, q_offset=99, topk=2)
    assert lib.ssa_block_sparse_attn_fwd(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                         None) == ssa.SSA_ERR_UNSUPPORTED


def test_backward_workspace_and_validation(lib):
    sh = good_shape()            # b=1, Hq=4, Hkv=2, 256 rows: 4 query / key blocks
    p = ctypes.byref(sh)
    rows = 4 * 4 * 64 * 4        # per-row LSE / D arrays: 4 heads x 4 query blocks x 64 rows, fp32
    piece = 2 * 64 * 64 * 4           # (dK, dV) partial of one key block: 2 x 64 x 64 fp32
    # block-sparse: a group (2 query heads) lists at most 2 * (1 + 2 + 2 + 2) = 14 pairs, so
    # 14 ranges; a partial per (range, key block) piece: 14 + 4 pieces per group
    parts = 2 * (14 + 4) * piece
    need = lib.ssa_workspace_bytes(p, ssa.SSA_OP_SPARSE_BWD)
    # + head bits and pair counts, pair starts: each under 256 bytes, padded to 256
    assert need == 2 * rows + 2 * 256 + parts
    # full: 2 * (4 + 2) = 12 pairs over the key units (blocks 0-1, 2-3) of a group, so 12
    # ranges and 12 + 2 pieces, each holding two key blocks
    need_full = lib.ssa_workspace_bytes(p, ssa.SSA_OP_FULL_BWD)
    assert need_full == 2 * rows + 256 + 2 * (12 + 2) * 2 * piece
    args = (FAKE,) * 10
    assert lib.ssa_block_sparse_attn_bwd(p, *args, FAKE, need - 1, None) == ssa.SSA_ERR_WORKSPACE
    assert lib.ssa_block_sparse_attn_bwd(p, *args, ctypes.c_void_p(0x10080), need, None) == ssa.SSA_ERR_INVALID_ARG
    assert b"workspace" in lib.ssa_last_error()
    assert lib.ssa_block_sparse_attn_bwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, need,
                                         None) == ssa.SSA_ERR_INVALID_ARG
    assert b"dout is NULL" in lib.ssa_last_error()
    assert lib.ssa_full_attn_bwd(p, FAKE, FAKE, FAKE, 3, 2, *((FAKE,) * 7), need, None) == ssa.SSA_ERR_INVALID_ARG
    # a slice never needs more workspace than the whole range
    assert lib.ssa_full_attn_bwd(p, FAKE, FAKE, FAKE, 2, 2, *((FAKE,) * 6), None, need_full,
                                 None) == ssa.SSA_ERR_INVALID_ARG
    assert b"workspace is NULL" in lib.ssa_last_error()
    # group-shared / per-head masks hold 32 heads per KV head at most
    wide = good_shape(n_q_heads=64, n_kv_heads=1)
    assert lib.ssa_block_sparse_attn_bwd(ctypes.byref(wide), *args, FAKE, 1 << 40, None) == ssa.SSA_ERR_UNSUPPORTED
    # a KV group with more than 2^31 - 1 (query head, query block, key block) pairs
    huge = good_shape(n_q_heads=32, n_kv_heads=1, seq_q=1 << 20, seq_kv=1 << 20)
    assert lib.ssa_full_attn_bwd(ctypes.byref(huge), FAKE, FAKE, FAKE, 0, (1 << 20) // 64, *((FAKE,) * 7), 1 << 40,
                                 None) == ssa.SSA_ERR_UNSUPPORTED
    assert b"too large" in lib.ssa_last_error()
    # the partials of a long sequence stay bounded by the ranges and key blocks
    long = good_shape(n_q_heads=32, n_kv_heads=2, seq_q=32768, seq_kv=32768, topk=16)
    assert lib.ssa_workspace_bytes(ctypes.byref(long), ssa.SSA_OP_SPARSE_BWD) < 1 << 30


def test_dash_route_validation(lib):
    p = ctypes.byref(good_shape())
    f = ctypes.c_float
    args = (FAKE, FAKE, None, None)
    for alpha, st in ((1.0, ssa.SSA_ERR_UNSUPPORTED), (2.5, ssa.SSA_ERR_UNSUPPORTED),
                      (float("nan"), ssa.SSA_ERR_INVALID_ARG)):
        assert lib.ssa_entmax_route(p, FAKE, f(alpha), f(1.0), f(1.0), *args) == st
        assert b"alpha" in lib.ssa_last_error()
    for gamma, sigma in ((-1.0, 1.0), (1.0, -0.5), (float("inf"), 1.0), (1.0, float("nan"))):
        assert lib.ssa_entmax_route(p, FAKE, f(1.5), f(gamma), f(sigma), *args) == ssa.SSA_ERR_INVALID_ARG
    assert lib.ssa_entmax_route(p, FAKE, f(1.5), f(1.0), f(1.0), FAKE, None, None, None) == ssa.SSA_ERR_INVALID_ARG
    assert b"block_bias is NULL" in lib.ssa_last_error()
    long = good_shape(seq_q=64 * 1025, seq_kv=64 * 1025)
    assert lib.ssa_entmax_route(ctypes.byref(long), FAKE, f(1.5), f(1.0), f(1.0), FAKE, FAKE, None,
                                None) == ssa.SSA_ERR_UNSUPPORTED
    # the biased forward: decode needs the decode workspace; the bias is required
    dec = good_shape(seq_q=1, seq_kv=300, q_offset=299)
    assert lib.ssa_block_sparse_attn_fwd_biased(ctypes.byref(dec), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                                                None) == ssa.SSA_ERR_WORKSPACE
    assert lib.ssa_block_sparse_attn_fwd_biased(p, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 0,
                                                None) == ssa.SSA_ERR_INVALID_ARG
    assert lib.ssa_block_summaries_learned(p, FAKE, None, FAKE, None) == ssa.SSA_ERR_INVALID_ARG
    assert b"qbar is NULL" in lib.ssa_last_error()


def test_empty_problems_launch_nothing(lib):
    # batch 0 or no query rows: SSA_OK with no HIP call (works without a GPU)
    for sh in (good_shape(batch=0), good_shape(seq_q=0, seq_kv=0)):
        p = ctypes.byref(sh)
        assert lib.ssa_block_scores(p, FAKE, FAKE, FAKE, 0, FAKE, None) == ssa.SSA_OK
        assert lib.ssa_select_topk(p, FAKE, FAKE, None) == ssa.SSA_OK
        assert lib.ssa_block_sparse_attn_fwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == ssa.SSA_OK
        assert lib.ssa_full_attn_fwd_dropped_mass(p, FAKE, FAKE, FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, None, 0,
                                                  None) == ssa.SSA_OK
        assert lib.ssa_select_topk_shared(p, FAKE, FAKE, None) == ssa.SSA_OK
        assert lib.ssa_block_sparse_attn_fwd_shared(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                                                    None) == ssa.SSA_OK
        assert lib.ssa_block_sparse_attn_bwd(p, *((FAKE,) * 11), 0, None) == ssa.SSA_OK
        assert lib.ssa_full_attn_bwd(p, FAKE, FAKE, FAKE, 0, 0, *((FAKE,) * 7), 0, None) == ssa.SSA_OK
    sh = good_shape()
    assert lib.ssa_full_attn_fwd_dropped_mass(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, 2, 0, FAKE, FAKE, FAKE,
                                              None, 0, None) == ssa.SSA_OK


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ssa.ssa_block_summaries(q)
