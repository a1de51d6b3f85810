"""CPU checks of the binding's argument validation: every wrapper refuses a
tensor whose dtype, shape or device does not match what its entry point reads
or writes for the given Shape, before anything reaches the library (meta
tensors: no memory, no GPU)."""
from __future__ import annotations

import pytest
import torch

from block_sparse_attention_kv_amd import ssa

B, HQ, HKV, N, D, K = 1, 4, 2, 256, 64, 3   # 4 query blocks


def t(*shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device="meta")


def shape(seq_q=N, topk=K):
    return ssa.Shape(batch=B, n_q_heads=HQ, n_kv_heads=HKV, seq_q=seq_q, seq_kv=N, q_offset=N - seq_q,
                     head_dim=D, block=64, topk=topk, causal=1, scale=0.0)


def good():
    return dict(q=t(B, HQ, N, D), k=t(B, HKV, N, D), v=t(B, HKV, N, D), idx=t(B, HQ, 4, K, dtype=torch.int32),
                idx_shared=t(B, HKV, 4, K, dtype=torch.int32), scores=t(B, HQ, 4, 4, dtype=torch.float32))


def refuses(fn, *args, match, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def test_correct_tensors_reach_the_device_check():
    g = good()
    # everything matches: the only refusal left is that meta tensors are not on the GPU
    refuses(ssa.ssa_block_sparse_attn_fwd, shape(), g["q"], g["k"], g["v"], g["idx"], match="GPU tensors only")


def test_sparse_forward_refusals():
    g = good()
    f = ssa.ssa_block_sparse_attn_fwd
    refuses(f, shape(), g["q"], g["k"], g["v"], g["idx"].to(torch.int64), match="block_idx has dtype")
    refuses(f, shape(), g["q"], t(B, 1, N, D), g["v"], g["idx"], match="k has shape")         # fewer KV heads
    refuses(f, shape(), g["q"], t(B, HKV, N - 64, D), g["v"], g["idx"], match="k has shape")  # shorter K
    refuses(f, shape(), g["q"].float(), g["k"], g["v"], g["idx"], match="q has dtype")
    refuses(f, shape(), g["q"], g["k"], g["v"], g["idx"], out=t(B, HQ, N - 1, D), match="out has shape")
    refuses(f, shape(), g["q"], g["k"], g["v"], g["idx"], lse=t(B, HQ, N), match="lse has dtype")
    refuses(f, shape(), g["q"], g["k"], g["v"], g["idx"], shared=True, match="block_idx has shape")
    refuses(f, shape(topk=K + 1), g["q"], g["k"], g["v"], g["idx"], match="block_idx has shape")
    refuses(f, shape(), g["q"], g["k"], g["v"], g["idx"], workspace=t(16, dtype=torch.int32),
            match="workspace has dtype")


def test_full_forward_refusals():
    g = good()
    f = ssa.ssa_full_attn_fwd_dropped_mass
    # a slice of two query blocks writes 128 rows
    refuses(f, shape(), g["q"], g["k"], g["v"], g["idx"], 1, 2, out=t(B, HQ, N, D), match="out has shape")
    refuses(f, shape(), g["q"], g["k"], g["v"], g["idx"], 1, 2, dropped=t(B, HQ, 64, dtype=torch.float32),
            match="dropped has shape")
    refuses(f, shape(), g["q"], g["k"], g["v"], g["idx_shared"], match="block_idx has shape")


def test_scores_topk_refusals():
    g = good()
    refuses(ssa.ssa_block_scores, shape(), g["q"], t(B, HKV, N, D, dtype=torch.float16), match="k has dtype")
    refuses(ssa.ssa_block_scores, shape(), g["q"], None, t(B, HKV, 3, D, dtype=torch.float32),
            match="k_summary has shape")
    refuses(ssa.ssa_select_topk, shape(), g["scores"], t(B, HQ, 4, K, dtype=torch.int64), match="idx has dtype")
    refuses(ssa.ssa_select_topk, shape(), g["scores"][:, :, :3], match="scores has shape")
    refuses(ssa.ssa_select_topk_shared, shape(), g["scores"], g["idx"], match="idx has shape")


def test_backward_and_other_refusals():
    g = good()
    o, lse, do = t(B, HQ, N, D), t(B, HQ, N, dtype=torch.float32), t(B, HQ, N, D)
    refuses(ssa.ssa_block_sparse_attn_bwd, shape(), g["q"], g["k"], g["v"], g["idx"], o, lse, do,
            dk=t(B, HKV, N, D - 8), match="dk has shape")
    refuses(ssa.ssa_block_sparse_attn_bwd, shape(), g["q"], g["k"], g["v"], g["idx"], o, lse.double(), do,
            match="lse has dtype")
    refuses(ssa.ssa_full_attn_bwd, shape(), g["q"], g["k"], g["v"], o[:, :, :128], lse, do, 2, 2,
            match="lse_full has shape")
    refuses(ssa.ssa_block_sparse_attn_fwd_early_stop, shape(), g["q"], g["k"], g["v"], g["scores"], g["idx"], 0.1,
            blocks_used=t(B, HQ, 4, dtype=torch.float32), match="blocks_used has dtype")
    refuses(ssa.ssa_entmax_route, shape(), g["scores"], 1.5, 1.0, 1.0, idx=g["idx"], match="idx has shape")
    refuses(ssa.ssa_block_sparse_attn_fwd_biased, shape(), g["q"], g["k"], g["v"], g["idx_shared"],
            t(B, HKV, 4, K, dtype=torch.bfloat16), match="block_bias has dtype")
    refuses(ssa.ssa_block_summaries_learned, g["k"], t(HKV, D + 1, dtype=torch.float32), match="qbar has shape")


def test_mixed_devices_refused():
    g = good()
    refuses(ssa.ssa_block_sparse_attn_fwd, shape(), g["q"], torch.empty((B, HKV, N, D), dtype=torch.bfloat16),
            g["v"], g["idx"], match="is on")
